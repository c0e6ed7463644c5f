// Per-page key summary for the quad score, built when a page is appended.
// AMASS (amass-kv 0.1.1 project page), "What is in the box" item 1: the quad
// selector keeps a tiny per-page summary with r' eigen-quantities instead of
// the per-key coordinates.  Per (physical page, KV head), over n valid keys:
//   mu = mean key, Xc = keys - mu, Gram = Xc Xc^T / n (n <= 32),
//   the top R eigenpairs of Gram in float32, lam descending,
//   w_j = Xc^T v_j / sqrt(n) (= sqrt(lam_j) u_j), zero when j > n-1 or
//   lam_j <= 1e-6 lam_1;
// stored as bfloat16 [mu, w_1..w_R] and float32 log n at the page's logical
// position (sequence, KV head, page), where the scorer streams them in order.
//
// One wave per (page, KV head).  The keys are centred into LDS once and the
// Gram comes from the float32 MFMA (16 x 16 tiles of X X^T), padded to P x P
// with zero rows (which only adds zero eigenvalues).  The top R eigenpairs are
// found without sweeping the whole spectrum, in registers: lane i (and its
// copies i + P, ...) holds row i of the Gram and of Q.
//   1. Householder reduction to tridiagonal form T = Q^T G Q (P - 2
//      reflections, each a rank-2 update of the trailing block), with Q
//      accumulated row by row;
//   2. the R largest eigenvalues of T by multisection on Sturm counts (the
//      lanes of a group evaluate the count at evenly spaced points of the
//      eigenvalue's bracket, so each round shrinks it lp + 1 times);
//   3. each eigenvector z of T from the twisted factorisation of T - lam I
//      (forward and backward LDL^T, twisted where |gamma| is smallest), its
//      Rayleigh quotient as the eigenvalue, modified Gram-Schmidt among the R
//      vectors, then u = Q z.
// A kept eigenvector that Gram-Schmidt leaves (almost) empty means an
// eigenvalue repeated inside the top R (T splits, and the twisted solves
// return the same vector); such a page is redone by cyclic Jacobi on the
// whole Gram with the round-robin ("circle") pair schedule, so the n/2
// rotations of a step are disjoint and a step is a set of independent 2x2
// block updates A <- J^T A J plus the column update V <- V J; sweeps stop when
// no off-diagonal element is above float32 noise (at most 16 sweeps).

#include "device.h"
#include "launch.h"

namespace kvs {

// Whether the pair (p, q) is rotated: its off-diagonal element is above
// float32 noise relative to the diagonal (tiny: an absolute floor).  The
// hardware square root (about 1 ulp) serves: only the same test must be used
// by the stop check and the steps.
__device__ __forceinline__ bool rotation_wanted(float app, float aqq, float apq, float tiny) {
  return fabsf(apq) > 1e-7f * __builtin_amdgcn_sqrtf(fabsf(app * aqq)) + tiny;
}

// Pair k of a step of the round-robin ("circle") schedule over m players:
// player 0 stays, players 1..m-1 rotate; p < q.
__device__ __forceinline__ void circle_pair(int step, int k, int m, int& p, int& q) {
  int x, y;
  if (k == 0) { x = 0; y = 1 + (step % (m - 1)); }
  else {
    x = 1 + ((step + k) % (m - 1));
    y = 1 + ((step + m - 1 - k) % (m - 1));
  }
  p = x < y ? x : y;
  q = x < y ? y : x;
}

// The rotation (c, s) that zeroes A[p][q] (smaller angle), or the identity
// when the pair fails the test.  Hardware reciprocal, square root and
// reciprocal square root: an ulp in c or s only changes how fast the sweeps
// converge.
__device__ __forceinline__ void jacobi_rotation(float app, float aqq, float apq, float tiny, float& c, float& s) {
  c = 1.f;
  s = 0.f;
  if (rotation_wanted(app, aqq, apq, tiny)) {
    const float theta = (aqq - app) * __builtin_amdgcn_rcpf(2.f * apq);
    const float t = (theta >= 0.f ? 1.f : -1.f) *
                    __builtin_amdgcn_rcpf(fabsf(theta) + __builtin_amdgcn_sqrtf(theta * theta + 1.f));
    c = __builtin_amdgcn_rsqf(t * t + 1.f);
    s = t * c;
  }
}

// A sweep whose pairs all fail the rotation test leaves A unchanged, so
// testing every pair on the current A at once decides the stop exactly as a
// sweep of no-op steps would (the block is one wave: a vote suffices).
template <int PS>
__device__ __forceinline__ bool jacobi_converged(float (*A)[PS + 1], int m, float tiny) {
  bool any = false;
  for (int idx = threadIdx.x; idx < m * m; idx += 64) {
    const int a = idx / m, b = idx - (idx / m) * m;
    if (a < b) any = any || rotation_wanted(A[a][a], A[b][b], A[a][b], tiny);
  }
  return !__any(any);
}

// Cyclic Jacobi on the m x m matrix A (LDS, symmetric), accumulating the
// rotations into V.  Any m: the n/2 rotations of a step are computed by the
// first lanes and handed to the update through LDS.
template <int PS>
__device__ __forceinline__ void jacobi_sweeps(float (*A)[PS + 1], float (*V)[PS + 1], float* rot_c, float* rot_s,
                                              int* rot_p, int* rot_q, int m, float tiny) {
  const int lane = threadIdx.x;
  const int half = m / 2;
  for (int sweep = 0; sweep < 16; ++sweep) {
    if (jacobi_converged<PS>(A, m, tiny)) break;
    for (int step = 0; step < m - 1; ++step) {
      if (lane < half) {
        int p, qq;
        circle_pair(step, lane, m, p, qq);
        float c, s;
        jacobi_rotation(A[p][p], A[qq][qq], A[p][qq], tiny, c, s);
        rot_p[lane] = p; rot_q[lane] = qq; rot_c[lane] = c; rot_s[lane] = s;
      }
      __syncthreads();
      for (int blk = lane; blk < half * half; blk += 64) {
        const int a = blk / half, bb = blk - a * half;
        const int pa = rot_p[a], qa = rot_q[a], pb = rot_p[bb], qb = rot_q[bb];
        const float ca = rot_c[a], sa = rot_s[a], cb = rot_c[bb], sb = rot_s[bb];
        const float b00 = A[pa][pb], b01 = A[pa][qb], b10 = A[qa][pb], b11 = A[qa][qb];
        const float t00 = ca * b00 - sa * b10, t01 = ca * b01 - sa * b11;
        const float t10 = sa * b00 + ca * b10, t11 = sa * b01 + ca * b11;
        A[pa][pb] = t00 * cb - t01 * sb;
        A[pa][qb] = t00 * sb + t01 * cb;
        A[qa][pb] = t10 * cb - t11 * sb;
        A[qa][qb] = t10 * sb + t11 * cb;
      }
      for (int idx = lane; idx < m * half; idx += 64) {
        const int r = idx / half, bb = idx - r * half;
        const int pb = rot_p[bb], qb = rot_q[bb];
        const float cb = rot_c[bb], sb = rot_s[bb];
        const float vp = V[r][pb], vq = V[r][qb];
        V[r][pb] = cb * vp - sb * vq;
        V[r][qb] = sb * vp + cb * vq;
      }
      __syncthreads();
    }
  }
}

// The same sweeps for a full page (m = PS = 16 or 32), with no LDS handoff:
// every lane owns the 2x2 blocks (a, bb) with bb = lane mod PS/2 fixed, and
// the V entries of the same column pair bb, and computes the rotations of its
// own pairs itself from the current A.  All of a step's LDS reads precede its
// writes (one wave: LDS serves them in program order), so each step is one
// round trip.  The rotations and updates are those of the general path (the
// compiler may fuse a product into a multiply-add differently, so the last
// bit can differ).
template <int PS>
__device__ __forceinline__ void jacobi_sweeps_full(float (*A)[PS + 1], float (*V)[PS + 1], float tiny) {
  constexpr int M = PS, H = PS / 2;
  constexpr int AS = 64 / H;           // the lane's blocks are rows a0, a0 + AS, ...
  constexpr int NB = H * H / 64;       // blocks per lane
  constexpr int NV = M * H / 64;       // V entry pairs per lane
  static_assert(64 % H == 0 && NB >= 1 && NV >= 1, "full-page Jacobi needs PS = 16 or 32");
  const int lane = threadIdx.x;
  const int bb = lane % H, a0 = lane / H;
  for (int sweep = 0; sweep < 16; ++sweep) {
    if (jacobi_converged<PS>(A, M, tiny)) break;
    for (int step = 0; step < M - 1; ++step) {
      int pb, qb, pa[NB], qa[NB];
      circle_pair(step, bb, M, pb, qb);
#pragma unroll
      for (int i = 0; i < NB; ++i) circle_pair(step, a0 + AS * i, M, pa[i], qa[i]);
      // reads
      const float bpp = A[pb][pb], bqq = A[qb][qb], bpq = A[pb][qb];
      float app[NB], aqq[NB], apq[NB], b00[NB], b01[NB], b10[NB], b11[NB], vp[NV], vq[NV];
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        app[i] = A[pa[i]][pa[i]]; aqq[i] = A[qa[i]][qa[i]]; apq[i] = A[pa[i]][qa[i]];
        b00[i] = A[pa[i]][pb]; b01[i] = A[pa[i]][qb]; b10[i] = A[qa[i]][pb]; b11[i] = A[qa[i]][qb];
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int r = a0 + AS * i;
        vp[i] = V[r][pb];
        vq[i] = V[r][qb];
      }
      // rotations of the lane's pairs
      float cb, sb;
      jacobi_rotation(bpp, bqq, bpq, tiny, cb, sb);
      // writes
#pragma unroll
      for (int i = 0; i < NB; ++i) {
        float ca, sa;
        jacobi_rotation(app[i], aqq[i], apq[i], tiny, ca, sa);
        const float t00 = ca * b00[i] - sa * b10[i], t01 = ca * b01[i] - sa * b11[i];
        const float t10 = sa * b00[i] + ca * b10[i], t11 = sa * b01[i] + ca * b11[i];
        A[pa[i]][pb] = t00 * cb - t01 * sb;
        A[pa[i]][qb] = t00 * sb + t01 * cb;
        A[qa[i]][pb] = t10 * cb - t11 * sb;
        A[qa[i]][qb] = t10 * sb + t11 * cb;
      }
#pragma unroll
      for (int i = 0; i < NV; ++i) {
        const int r = a0 + AS * i;
        V[r][pb] = cb * vp[i] - sb * vq[i];
        V[r][qb] = sb * vp[i] + cb * vq[i];
      }
      __syncthreads();
    }
  }
}

// Gram / n of the centred keys X (rows past n are zero) into A, on the float32
// MFMA: a 16 x 16 tile of X X^T takes D/4 steps of 16x16x4, lane l feeding
// X[row l%16][4 st + l/16] of both row blocks.  One writer per symmetric pair,
// so A is exactly symmetric.
template <int D, int PS>
__device__ __forceinline__ void gram_mfma(const float (*X)[D + 1], float (*A)[PS + 1], float inv_n) {
  typedef float f32x4v __attribute__((ext_vector_type(4)));
  constexpr int NT16 = PS / 16;
  const int lane = threadIdx.x;
  const int r16 = lane & 15, kq = lane >> 4;
#pragma unroll
  for (int ta = 0; ta < NT16; ++ta)
#pragma unroll
    for (int tb = ta; tb < NT16; ++tb) {
      f32x4v acc[4] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
#pragma unroll
      for (int st = 0; st < D / 4; ++st) {
        const float xa = X[16 * ta + r16][4 * st + kq];
        const float xb = X[16 * tb + r16][4 * st + kq];
        acc[st & 3] = __builtin_amdgcn_mfma_f32_16x16x4f32(xa, xb, acc[st & 3], 0, 0, 0);
      }
      const f32x4v t = (acc[0] + acc[1]) + (acc[2] + acc[3]);
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int ia = 16 * ta + 4 * kq + r, jb = 16 * tb + r16;
        if (ta < tb || ia <= jb) {
          const float v = t[r] * inv_n;
          A[ia][jb] = v;
          A[jb][ia] = v;
        }
      }
    }
}

// Sum over lanes 0..PS-1 of a layout in which lanes repeat every PS (16 or
// 32): DPP inside 16-lane rows, then across the row pair.  Uniform result.
template <int PS>
__device__ __forceinline__ float copy_sum(float x) {
  auto add = [](int a, int b) { return __float_as_int(__int_as_float(a) + __int_as_float(b)); };
  int v = __float_as_int(x);
  v = add(v, dpp<0x111, 0xF>(0, v));   // row_shr:1
  v = add(v, dpp<0x112, 0xF>(0, v));   // row_shr:2
  v = add(v, dpp<0x114, 0xF>(0, v));   // row_shr:4
  v = add(v, dpp<0x118, 0xF>(0, v));   // row_shr:8
  if constexpr (PS == 32) v = add(v, dpp<0x142, 0xA>(0, v));   // row_bcast:15
  return __int_as_float(__builtin_amdgcn_readlane(v, PS - 1));
}

// Householder reduction of the symmetric PS x PS matrix whose row i sits in
// a[] of the lanes i, i + PS, ...: T = Q^T A Q tridiagonal with diagonal d
// and off-diagonal e (uniform), Q = H_0 .. H_{PS-3} accumulated row-wise in
// qr[].  Reflection k takes v over rows k+1.. (v_{k+1} = x_{k+1} - alpha),
// beta = 2 / |v|^2 = 1 / (sig2 - x_{k+1} alpha), and the trailing block gets
// A <- A - v q^T - q v^T with p = beta A v, q = p - (beta/2)(p.v) v.  A column
// already zero below the subdiagonal (to tiny2) is left alone.
template <int PS>
__device__ __forceinline__ void householder_rows(float (&a)[PS], float (&qr)[PS], float (&d)[PS], float (&e)[PS],
                                                 float tiny2) {
  const int i = threadIdx.x & (PS - 1);
#pragma unroll
  for (int j = 0; j < PS; ++j) qr[j] = i == j ? 1.f : 0.f;
#pragma unroll
  for (int k = 0; k + 2 < PS; ++k) {
    const float xi = i > k ? a[k] : 0.f;
    const float sig2 = copy_sum<PS>(xi * xi);
    const float x0 = readlane_f(a[k], k + 1);
    d[k] = readlane_f(a[k], k);
    if (!(sig2 - x0 * x0 > tiny2)) {   // uniform
      e[k] = x0;
      continue;
    }
    const float sg = __builtin_amdgcn_sqrtf(sig2);
    const float alpha = x0 >= 0.f ? -sg : sg;
    const float bt = __builtin_amdgcn_rcpf(sig2 - x0 * alpha);
    e[k] = alpha;
    const float vi = i == k + 1 ? x0 - alpha : xi;
    float vj[PS];
#pragma unroll
    for (int j = k + 1; j < PS; ++j) vj[j] = j == k + 1 ? x0 - alpha : readlane_f(a[k], j);
    float p = 0.f, qv = 0.f;
#pragma unroll
    for (int j = k + 1; j < PS; ++j) {
      p = fmaf(a[j], vj[j], p);
      qv = fmaf(qr[j], vj[j], qv);
    }
    p = i > k ? p * bt : 0.f;
    qv *= bt;
    const float K = 0.5f * bt * copy_sum<PS>(p * vi);
    const float qi = p - K * vi;
#pragma unroll
    for (int j = k + 1; j < PS; ++j) {
      const float qj = readlane_f(qi, j);
      a[j] = fmaf(-vi, qj, fmaf(-qi, vj[j], a[j]));
      qr[j] = fmaf(-qv, vj[j], qr[j]);
    }
  }
  d[PS - 2] = readlane_f(a[PS - 2], PS - 2);
  d[PS - 1] = readlane_f(a[PS - 1], PS - 1);
  e[PS - 2] = readlane_f(a[PS - 2], PS - 1);
  e[PS - 1] = 0.f;
}

// The R (1, 2, 4 or 8) largest eigenpairs of the tridiagonal T (d, e) whose
// Householder product Q is in qr[] (row i = lane mod PS).  Returns
// u[j] = (Q z_j)_i in lane i and lam[j] (uniform); false when an eigenvector
// that the summary keeps (j + 1 <= kept and lam_j above 1e-6 lam_0) is, to
// half its length, a combination of the ones before it (an eigenvalue
// repeated inside the top R).
template <int PS>
__device__ __forceinline__ bool tridiag_top_eigen(const float (&d)[PS], const float (&e)[PS], const float (&qr)[PS],
                                                  int R, int kept, float (&u)[8], float (&lam)[8]) {
  const int lane = threadIdx.x;
  float e2[PS];
#pragma unroll
  for (int j = 0; j < PS; ++j) e2[j] = e[j] * e[j];
  float glo = INFINITY, ghi = -INFINITY;
#pragma unroll
  for (int j = 0; j < PS; ++j) {
    const float r = fabsf(e[j]) + (j > 0 ? fabsf(e[j - 1]) : 0.f);
    glo = fminf(glo, d[j] - r);
    ghi = fmaxf(ghi, d[j] + r);
  }
  {
    const float span = fmaxf(ghi - glo, fabsf(ghi) * 1e-6f + 1e-30f);
    glo -= 1e-6f * span;
    ghi += 1e-6f * span;
  }
  // Pivots of the LDL^T recurrences use the reciprocal clamped to +-1e30: a
  // zero pivot (+0 or -0) acts as a pivot of that sign and size, so the next
  // pivot is +-inf or huge, never NaN, even where e_j = 0 (T splits).
  auto rc = [](float x) { return __builtin_amdgcn_fmed3f(__builtin_amdgcn_rcpf(x), -1e30f, 1e30f); };

  // 1. multisection: lp lanes per eigenvalue t (index PS-1-t ascending) count
  //    the eigenvalues below lp evenly spaced points of its bracket
  const int lp = 64 / R;
  const int t = lane / lp, l = lane - t * lp;
  const int target = PS - 1 - t;
  const float step_den = 1.f / (float)(lp + 1);
  float blo = glo, bhi = ghi;
  const int rounds = lp >= 32 ? 5 : (lp >= 16 ? 6 : 7);
  for (int rd = 0; rd < rounds; ++rd) {
    const float w = bhi - blo;
    const float sigma = blo + w * ((float)(l + 1) * step_den);
    // negative pivots, counted by sign bit (-0 counts as negative, as its reciprocal does)
    float q = d[0] - sigma;
    unsigned c = __float_as_uint(q) >> 31;
#pragma unroll
    for (int j = 1; j < PS; ++j) {
      q = fmaf(-e2[j - 1], rc(q), d[j] - sigma);
      c += __float_as_uint(q) >> 31;
    }
    const unsigned long long ball = __ballot((int)c >= target + 1);
    const unsigned long long gm = lp == 64 ? ball : (ball >> (t * lp)) & ((1ull << lp) - 1ull);
    if (gm) {
      const int f = __ffsll((long long)gm) - 1;
      const float nhi = blo + w * ((float)(f + 1) * step_den);
      blo = f > 0 ? blo + w * ((float)f * step_den) : blo;
      bhi = nhi;
    } else {
      blo = blo + w * ((float)lp * step_den);
    }
  }
  // lane t (< R) takes eigenvalue t's estimate
  const float lm = __shfl(0.5f * (blo + bhi), (lane * lp) & 63);

  // 2. twisted factorisation of T - lm I: forward pivots Dp, backward Dm,
  //    twist index r where |gamma_r| = |Dp_r + Dm_r - (d_r - lm)| is least;
  //    z_r = 1, z_i = -(e_i / Dp_i) z_{i+1} below, z_i = -(e_{i-1} / Dm_i) z_{i-1} above
  float Dp[PS], Ub[PS];
  Dp[0] = d[0] - lm;
#pragma unroll
  for (int j = 0; j + 1 < PS; ++j) Dp[j + 1] = fmaf(-e[j] * rc(Dp[j]), e[j], d[j + 1] - lm);
  float Dm = d[PS - 1] - lm;
  float best = fabsf(Dp[PS - 1]);
  int r = PS - 1;
#pragma unroll
  for (int j = PS - 2; j >= 0; --j) {
    Ub[j] = e[j] * rc(Dm);
    Dm = fmaf(-Ub[j], e[j], d[j] - lm);
    const float gam = fabsf(Dp[j] + Dm - (d[j] - lm));
    if (gam < best) {
      best = gam;
      r = j;
    }
  }
  float z[PS];
  {
    float zd = r == PS - 1 ? 1.f : 0.f;
    z[PS - 1] = zd;
#pragma unroll
    for (int j = PS - 2; j >= 0; --j) {
      zd = j == r ? 1.f : -(e[j] * rc(Dp[j])) * zd;
      z[j] = zd;
    }
    float zu = r == 0 ? 1.f : 0.f;
#pragma unroll
    for (int j = 1; j < PS; ++j) {
      zu = j == r ? 1.f : -Ub[j - 1] * zu;
      if (j > r) z[j] = zu;
    }
  }
  // normalise; the Rayleigh quotient z^T T z is the eigenvalue estimate
  float nz = 0.f;
#pragma unroll
  for (int j = 0; j < PS; ++j) nz = fmaf(z[j], z[j], nz);
  const float inz = __builtin_amdgcn_rsqf(fmaxf(nz, 1e-37f));
#pragma unroll
  for (int j = 0; j < PS; ++j) z[j] *= inz;
  float rq = 0.f;
#pragma unroll
  for (int j = 0; j < PS; ++j) {
    float tz = d[j] * z[j];
    if (j > 0) tz = fmaf(e[j - 1], z[j - 1], tz);
    if (j + 1 < PS) tz = fmaf(e[j], z[j + 1], tz);
    rq = fmaf(z[j], tz, rq);
  }
#pragma unroll
  for (int j = 0; j < 8; ++j) lam[j] = j < R ? readlane_f(rq, j) : 0.f;

  // 3. modified Gram-Schmidt over lanes 0..R-1, z_s broadcast to the lanes after it
  bool good = true;
  const float lam_floor = 1e-6f * fmaxf(lam[0], 0.f);
#pragma unroll
  for (int s2 = 0; s2 < 8; ++s2) {
    if (s2 >= R) break;
    float n2 = 0.f;
#pragma unroll
    for (int j = 0; j < PS; ++j) n2 = fmaf(z[j], z[j], n2);
    const float n2s = readlane_f(n2, s2);
    if (!(n2s >= 0.25f) && s2 + 1 <= kept && lam[s2] > lam_floor) good = false;
    const float sc = __builtin_amdgcn_rsqf(fmaxf(n2s, 1e-37f));
    float zs[PS];
    float dot = 0.f;
#pragma unroll
    for (int j = 0; j < PS; ++j) {
      zs[j] = readlane_f(z[j], s2) * sc;
      dot = fmaf(z[j], zs[j], dot);
    }
    dot = lane > s2 ? dot : 0.f;
#pragma unroll
    for (int j = 0; j < PS; ++j) z[j] = lane == s2 ? zs[j] : fmaf(-dot, zs[j], z[j]);
  }

  // 4. back-transform: u_j = Q z_j, row i of Q in this lane
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    float acc = 0.f;
    if (j < R) {
#pragma unroll
      for (int k = 0; k < PS; ++k) acc = fmaf(qr[k], readlane_f(z[k], j), acc);
    }
    u[j] = acc;
  }
  return good;
}

template <int D, int PS, bool F16>
__global__ __launch_bounds__(64) void summary_build_kernel(const uint16_t* __restrict__ k16,
                                                           const int32_t* __restrict__ block_table,
                                                           int max_pages,
                                                           const int32_t* __restrict__ entries,
                                                           const int32_t* __restrict__ n_valid,
                                                           int Hkv, int R, uint16_t* __restrict__ summary,
                                                           float* __restrict__ log_n) {
  constexpr int CPL = D / 64;   // columns per lane
  __shared__ float X[PS][D + 1];
  __shared__ float A[PS][PS + 1];
  __shared__ float V[PS][PS + 1];
  __shared__ float rot_c[PS / 2], rot_s[PS / 2];
  __shared__ int rot_p[PS / 2], rot_q[PS / 2];
  __shared__ int order[PS];

  const int lane = threadIdx.x;
  const int i = blockIdx.x / Hkv, g = blockIdx.x - (blockIdx.x / Hkv) * Hkv;
  const int sb = entries[2 * i], sp = entries[2 * i + 1];   // sequence, logical page
  const int phys = block_table[(size_t)sb * max_pages + sp];
  int nv = n_valid[i];
  nv = nv < 0 ? 0 : (nv > PS ? PS : nv);
  const uint16_t* src = k16 + ((size_t)phys * Hkv + g) * PS * D;
  uint16_t* dst = summary + (((size_t)sb * Hkv + g) * max_pages + sp) * (size_t)(1 + R) * D;
  float* ln = log_n + (size_t)sb * max_pages + sp;

  if (nv == 0) {
    for (int e = lane; e < (1 + R) * D; e += 64) dst[e] = 0;
    if (g == 0 && lane == 0) *ln = -INFINITY;
    return;
  }

  // mean (token order, float32) and centred keys.  Every slot of a page is
  // allocated, so all PS keys are requested at once and slots past n masked.
  uint16_t raw[CPL][PS];
#pragma unroll
  for (int c = 0; c < CPL; ++c)
#pragma unroll
    for (int t = 0; t < PS; ++t) raw[c][t] = src[(size_t)t * D + lane + 64 * c];
  float mu[CPL];
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = lane + 64 * c;
    float s = 0.f;
#pragma unroll
    for (int t = 0; t < PS; ++t)
      if (t < nv) s += h16_to_f32<F16>(raw[c][t]);
    mu[c] = s / (float)nv;
    dst[e] = (uint16_t)f32_to_bf16_rne(mu[c]);
#pragma unroll
    for (int t = 0; t < PS; ++t) X[t][e] = t < nv ? h16_to_f32<F16>(raw[c][t]) - mu[c] : 0.f;
  }
  __syncthreads();

  const int row = lane & (PS - 1);
  const float inv_n = 1.f / (float)nv;
  gram_mfma<D, PS>(X, A, inv_n);
  __syncthreads();
  const float trace = copy_sum<PS>(A[row][row]);
  const float tiny = 1e-12f * trace;
  float u[8], lam[8];
  bool good;
  {
    float a[PS], qr[PS], d[PS], e[PS];
#pragma unroll
    for (int j = 0; j < PS; ++j) a[j] = A[row][j];
    householder_rows<PS>(a, qr, d, e, tiny * tiny);
    good = tridiag_top_eigen<PS>(d, e, qr, R, nv - 1, u, lam);   // w_j is kept only for j + 1 <= n - 1
  }
  if (!good) {
    // an eigenvalue repeated inside the top R: cyclic Jacobi on the whole Gram
    int m = nv + (nv & 1);
    if (m < 2) m = 2;
    __syncthreads();
    gram_mfma<D, PS>(X, A, inv_n);
    __syncthreads();
    for (int idx = lane; idx < m * m; idx += 64) {
      const int a = idx / m, bb = idx - a * m;
      V[a][bb] = a == bb ? 1.f : 0.f;
    }
    __syncthreads();
    if (m == PS) jacobi_sweeps_full<PS>(A, V, tiny);
    else jacobi_sweeps<PS>(A, V, rot_c, rot_s, rot_p, rot_q, m, tiny);
    // eigenvalues descending (ties by index) -> order[rank] = column
    if (lane < m) {
      const float lj = A[lane][lane];
      int pos = 0;
      for (int j = 0; j < m; ++j) {
        const float li = A[j][j];
        pos += (li > lj) || (li == lj && j < lane);
      }
      order[pos] = lane;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const int col = j < m ? order[j] : 0;
      lam[j] = j < R && j < m ? A[col][col] : 0.f;
      u[j] = j < R && j < m && row < m ? V[row][col] : 0.f;
    }
  }

  // w_j = Xc^T u_j / sqrt(n): keys of the lane's columns from LDS, u_j[t]
  // broadcast from lane t
  const float lam1 = fmaxf(lam[0], 0.f);
  const float inv_sqrt_n = 1.f / sqrtf((float)nv);
  float xv[PS][CPL];
#pragma unroll
  for (int t = 0; t < PS; ++t)
#pragma unroll
    for (int c = 0; c < CPL; ++c) xv[t][c] = X[t][lane + 64 * c];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    if (j >= R) break;   // uniform
    const bool zero = (j + 1 > nv - 1) || !(fmaxf(lam[j], 0.f) > 1e-6f * lam1);
    float w[CPL];
#pragma unroll
    for (int c = 0; c < CPL; ++c) w[c] = 0.f;
#pragma unroll
    for (int t = 0; t < PS; ++t) {
      const float ut = readlane_f(u[j], t);
#pragma unroll
      for (int c = 0; c < CPL; ++c) w[c] = fmaf(xv[t][c], ut, w[c]);
    }
#pragma unroll
    for (int c = 0; c < CPL; ++c)
      dst[(size_t)(1 + j) * D + lane + 64 * c] = (uint16_t)f32_to_bf16_rne(zero ? 0.f : w[c] * inv_sqrt_n);
  }
  if (g == 0 && lane == 0) *ln = logf((float)nv);
}

hipError_t launch_summary_build(const kv_layout& L, const void* k16, const int32_t* block_table,
                                int max_pages, const int32_t* entries, const int32_t* n_valid, int n,
                                void* summary, float* log_n, hipStream_t st) {
  const dim3 grid(n * L.num_kv_heads);
  const bool f16 = L.kv_dtype == KV_F16;
  const uint16_t* k = (const uint16_t*)k16;
  uint16_t* s = (uint16_t*)summary;
#define KVS_SB(D_, PS_, F_) hipLaunchKernelGGL((summary_build_kernel<D_, PS_, F_>), grid, dim3(64), 0, st, \
                                               k, block_table, max_pages, entries, n_valid, L.num_kv_heads, \
                                               L.rank, s, log_n)
  if (L.head_dim == 64) {
    if (L.page_size == 16) { if (f16) KVS_SB(64, 16, true); else KVS_SB(64, 16, false); }
    else { if (f16) KVS_SB(64, 32, true); else KVS_SB(64, 32, false); }
  } else {
    if (L.page_size == 16) { if (f16) KVS_SB(128, 16, true); else KVS_SB(128, 16, false); }
    else { if (f16) KVS_SB(128, 32, true); else KVS_SB(128, 32, false); }
  }
#undef KVS_SB
  return hipGetLastError();
}

}  // namespace kvs
