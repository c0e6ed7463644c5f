// Per-page key summary for the quad score, built when a page is appended.
// AMASS (amass-kv 0.1.1 project page), "What is in the box" item 1: the quad
// selector keeps a tiny per-page summary with r' eigen-quantities instead of
// the per-key coordinates.  Per (physical page, KV head), over n valid keys:
//   mu = mean key, Xc = keys - mu, Gram = Xc Xc^T / n (n <= 32),
//   eigenpairs of Gram by cyclic Jacobi in float32, lam descending,
//   w_j = Xc^T v_j / sqrt(n) (= sqrt(lam_j) u_j), zero when j > n-1 or
//   lam_j <= 1e-6 lam_1;
// stored as bfloat16 [mu, w_1..w_R] and float32 log n at the page's logical
// position (sequence, KV head, page), where the scorer streams them in order.
//
// One wave per (page, KV head).  The keys are centred into LDS once; the
// n x n Gram comes from LDS dot products; Jacobi runs with the round-robin
// ("circle") pair schedule, so the n/2 rotations of a step are disjoint and
// the whole step is a set of independent 2x2 block updates A <- J^T A J plus
// the column update V <- V J.  A sweep applies every pair once; sweeps stop
// when no off-diagonal element is above float32 noise (at most 16 sweeps);
// that test is one pass over all pairs before each sweep.

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
  int m = nv + (nv & 1);
  if (m < 2) m = 2;
  const int half = m / 2;
  __syncthreads();

  // Gram / n
  const float inv_n = 1.f / (float)nv;
  for (int idx = lane; idx < m * m; idx += 64) {
    const int a = idx / m, bb = idx - a * m;
    if (a <= bb) {
      float s = 0.f;
      for (int e = 0; e < D; ++e) s += X[a][e] * X[bb][e];
      s *= inv_n;
      A[a][bb] = s;
      A[bb][a] = s;
    }
    V[a][bb] = a == bb ? 1.f : 0.f;
  }
  __syncthreads();
  float trace = 0.f;
  for (int a = 0; a < m; ++a) trace += A[a][a];
  const float tiny = 1e-12f * trace;

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
  const float lam1 = fmaxf(A[order[0]][order[0]], 0.f);
  const float inv_sqrt_n = 1.f / sqrtf((float)nv);
  for (int j = 0; j < R; ++j) {
    float lam = 0.f;
    int colj = 0;
    if (j < m) { colj = order[j]; lam = fmaxf(A[colj][colj], 0.f); }
    const bool zero = (j + 1 > nv - 1) || !(lam > 1e-6f * lam1);
#pragma unroll
    for (int c = 0; c < CPL; ++c) {
      const int e = lane + 64 * c;
      float w = 0.f;
      if (!zero) {
        for (int t = 0; t < nv; ++t) w += X[t][e] * V[t][colj];
        w *= inv_sqrt_n;
      }
      dst[(size_t)(1 + j) * D + e] = (uint16_t)f32_to_bf16_rne(w);
    }
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
