// Shared-basis summaries, built at prefill / page append.  AMASS (amass-kv
// 0.1.1 project page), "What is in the box" item 1: the quad summary keeps
// only r' eigen-quantities per page.  Here the r' directions are shared by
// every page of a (sequence, KV head) row and each page keeps its mean and
// the variances of its keys along them:
//   row basis : u_1..u_r' = top eigenvectors of the population covariance of
//               the row's valid keys (float32, rows descending, each row's
//               largest-magnitude entry positive)
//   page      : mu = mean key (bfloat16), lam_j = mean of (u_j.(k - mu))^2
//               about the float32 mean (float32), log n (float32)
//
// Basis, two kernels:
//  * basis_cov_kernel: one block per (row, chunk of pages).  Keys are staged
//    128 tokens at a time in LDS; each thread accumulates an 8 x 8 block of
//    sum (k - s)(k - s)^T about a shift s (the chunk's first key), so the
//    chunk's (n, mean, M2) come out without cancellation against a large mean.
//  * basis_eigen_kernel: one block per row.  Chunk statistics are merged in
//    chunk order with the pairwise (Chan et al.) update, C = M2 / n goes to
//    LDS, and cyclic Jacobi with the round-robin ("circle") pair schedule
//    diagonalises it: the d/2 rotations of a step are disjoint, so a step is a
//    set of independent 2x2 block updates A <- J^T A J and V <- V J.  Sweeps
//    stop when no off-diagonal element is above float32 noise (at most 24).
// Page statistics: one wave per (page, KV head), keys centred into LDS, then
// one (token, direction) projection per lane and a DPP sum per direction.

#include "device.h"
#include "launch.h"

namespace kvs {

constexpr int kCovStage = 128;   // tokens staged in LDS at a time

template <int D, bool F16>
__global__ __launch_bounds__((D / 8) * (D / 8)) void basis_cov_kernel(
    const uint16_t* __restrict__ k16, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int Hkv, int P, int max_pages, int chunk_pages, int n_chunks,
    float* __restrict__ part) {
  constexpr int NB = D / 8;           // 8-wide blocks per dimension
  constexpr int NT = NB * NB;         // threads
  __shared__ uint16_t X[kCovStage][D + 8];   // staged 16-bit keys (padded rows)
  __shared__ float shift[D], S1s[D];

  const int c = blockIdx.x, row = blockIdx.y;
  const int b = row / Hkv, g = row - b * Hkv;
  const int tid = threadIdx.x;
  const int bi = tid / NB, bj = tid - bi * NB;
  int L = seq_lens[b];
  L = L < 0 ? 0 : (L > max_pages * P ? max_pages * P : L);
  const int t0 = c * chunk_pages * P;
  const int t1 = t0 + chunk_pages * P < L ? t0 + chunk_pages * P : L;
  const int n = t1 > t0 ? t1 - t0 : 0;
  float* dst = part + ((size_t)row * n_chunks + c) * (size_t)(1 + D + D * D);

  auto key_ptr = [&](int t) {
    const int p = t / P;
    const int phys = block_table[(size_t)b * max_pages + p];
    return k16 + (((size_t)phys * Hkv + g) * P + (t - p * P)) * D;
  };
  if (n > 0) {
    const uint16_t* s0 = key_ptr(t0);
    for (int e = tid; e < D; e += NT) shift[e] = h16_to_f32<F16>(s0[e]);
  }
  __syncthreads();
  float sr[8], sc[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) { sr[i] = n > 0 ? shift[8 * bi + i] : 0.f; sc[i] = n > 0 ? shift[8 * bj + i] : 0.f; }

  float acc[8][8];
  float s1[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    s1[i] = 0.f;
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = 0.f;
  }
  for (int base = t0; base < t1; base += kCovStage) {
    const int cnt = t1 - base < kCovStage ? t1 - base : kCovStage;
    // stage: thread tid copies tokens tid, tid + NT, ... of this stage
    for (int t = tid; t < cnt; t += NT) {
      const uint16_t* src = key_ptr(base + t);
#pragma unroll
      for (int e = 0; e < D; e += 8) *reinterpret_cast<u32x4_t*>(&X[t][e]) = ld16(src + e);
    }
    __syncthreads();
    for (int t = 0; t < cnt; ++t) {
      const u32x4_t ra = *reinterpret_cast<const u32x4_t*>(&X[t][8 * bi]);
      const u32x4_t rb = *reinterpret_cast<const u32x4_t*>(&X[t][8 * bj]);
      float xa[8], xb[8];
#pragma unroll
      for (int w = 0; w < 4; ++w) {
        xa[2 * w] = lo16<F16>(ra[w]) - sr[2 * w];
        xa[2 * w + 1] = hi16<F16>(ra[w]) - sr[2 * w + 1];
        xb[2 * w] = lo16<F16>(rb[w]) - sc[2 * w];
        xb[2 * w + 1] = hi16<F16>(rb[w]) - sc[2 * w + 1];
      }
      if (bj == 0) {
#pragma unroll
        for (int i = 0; i < 8; ++i) s1[i] += xa[i];
      }
#pragma unroll
      for (int i = 0; i < 8; ++i)
#pragma unroll
        for (int j = 0; j < 8; ++j) acc[i][j] = __builtin_fmaf(xa[i], xb[j], acc[i][j]);
    }
    __syncthreads();
  }
  if (bj == 0) {
#pragma unroll
    for (int i = 0; i < 8; ++i) S1s[8 * bi + i] = s1[i];
  }
  __syncthreads();
  // chunk statistics: mean = s + S1 / n, M2 = S2 - S1 S1^T / n
  const float inv_n = n > 0 ? 1.f / (float)n : 0.f;
  if (tid == 0) dst[0] = (float)n;
  for (int e = tid; e < D; e += NT) dst[1 + e] = n > 0 ? shift[e] + S1s[e] * inv_n : 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const float a = S1s[8 * bi + i];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      const float m2 = n > 0 ? acc[i][j] - a * S1s[8 * bj + j] * inv_n : 0.f;
      dst[1 + D + (size_t)(8 * bi + i) * D + 8 * bj + j] = m2;
    }
  }
}

template <int D>
__global__ __launch_bounds__((D / 8) * (D / 8)) void basis_eigen_kernel(const float* __restrict__ part,
                                                                          int n_chunks, int R,
                                                                          float* __restrict__ basis,
                                                                          float* __restrict__ mean_out) {
  constexpr int NB = D / 8;
  constexpr int NT = NB * NB;
  constexpr int HALF = D / 2;
  __shared__ float A[D][D + 1];
  __shared__ float V[D][D + 1];
  __shared__ float mean[D], dmean[D];
  __shared__ float rot_c[HALF], rot_s[HALF];
  __shared__ int rot_p[HALF], rot_q[HALF];
  __shared__ int order[D];
  __shared__ int n_rot;

  const int row = blockIdx.x;
  const int tid = threadIdx.x;
  const int bi = tid / NB, bj = tid - bi * NB;
  const float* src = part + (size_t)row * n_chunks * (size_t)(1 + D + D * D);

  // merge the chunk statistics in chunk order
  float M[8][8];
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) M[i][j] = 0.f;
  for (int e = tid; e < D; e += NT) mean[e] = 0.f;
  float n = 0.f;
  __syncthreads();
  for (int c = 0; c < n_chunks; ++c) {
    const float* pc = src + (size_t)c * (1 + D + D * D);
    const float nc = pc[0];
    if (!(nc > 0.f)) continue;
    const float tot = n + nc;
    const float f = nc / tot, w = n * nc / tot;
    for (int e = tid; e < D; e += NT) dmean[e] = pc[1 + e] - mean[e];
    __syncthreads();
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      const float di = dmean[8 * bi + i];
#pragma unroll
      for (int j = 0; j < 8; ++j)
        M[i][j] += pc[1 + D + (size_t)(8 * bi + i) * D + 8 * bj + j] + di * dmean[8 * bj + j] * w;
    }
    for (int e = tid; e < D; e += NT) mean[e] += dmean[e] * f;
    n = tot;
    __syncthreads();
  }
  if (mean_out)
    for (int e = tid; e < D; e += NT) mean_out[(size_t)row * D + e] = mean[e];
  const float inv_n = n > 0.f ? 1.f / n : 0.f;
#pragma unroll
  for (int i = 0; i < 8; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) {
      A[8 * bi + i][8 * bj + j] = M[i][j] * inv_n;
      V[8 * bi + i][8 * bj + j] = (8 * bi + i) == (8 * bj + j) ? 1.f : 0.f;
    }
  __syncthreads();
  float trace = 0.f;
  for (int a = 0; a < D; ++a) trace += A[a][a];
  const float tiny = 1e-12f * trace;

  for (int sweep = 0; sweep < 24; ++sweep) {
    if (tid == 0) n_rot = 0;
    __syncthreads();
    for (int step = 0; step < D - 1; ++step) {
      if (tid < HALF) {
        // circle method: player 0 fixed, players 1..D-1 rotate
        int x, y;
        if (tid == 0) { x = 0; y = 1 + (step % (D - 1)); }
        else {
          x = 1 + ((step + tid) % (D - 1));
          y = 1 + ((step + D - 1 - tid) % (D - 1));
        }
        const int p = x < y ? x : y, qq = x < y ? y : x;
        const float app = A[p][p], aqq = A[qq][qq], apq = A[p][qq];
        float cs = 1.f, sn = 0.f;
        if (fabsf(apq) > 1e-7f * sqrtf(fabsf(app * aqq)) + tiny) {
          const float theta = (aqq - app) / (2.f * apq);
          const float t = (theta >= 0.f ? 1.f : -1.f) / (fabsf(theta) + sqrtf(theta * theta + 1.f));
          cs = 1.f / sqrtf(t * t + 1.f);
          sn = t * cs;
          atomicAdd(&n_rot, 1);
        }
        rot_p[tid] = p; rot_q[tid] = qq; rot_c[tid] = cs; rot_s[tid] = sn;
      }
      __syncthreads();
      for (int blk = tid; blk < HALF * HALF; blk += NT) {
        const int a = blk / HALF, bb = blk - a * HALF;
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
      for (int idx = tid; idx < D * HALF; idx += NT) {
        const int r = idx / HALF, bb = idx - r * HALF;
        const int pb = rot_p[bb], qb = rot_q[bb];
        const float cb = rot_c[bb], sb = rot_s[bb];
        const float vp = V[r][pb], vq = V[r][qb];
        V[r][pb] = cb * vp - sb * vq;
        V[r][qb] = sb * vp + cb * vq;
      }
      __syncthreads();
    }
    const int applied = n_rot;
    __syncthreads();
    if (applied == 0) break;
  }

  // eigenvalues descending (ties by index) -> order[rank] = column
  for (int j = tid; j < D; j += NT) order[j] = j;
  __syncthreads();
  for (int j = tid; j < D; j += NT) {
    const float lj = A[j][j];
    int pos = 0;
    for (int i = 0; i < D; ++i) {
      const float li = A[i][i];
      pos += (li > lj) || (li == lj && i < j);
    }
    order[pos] = j;
  }
  __syncthreads();
  // rows of the basis: eigenvector columns scaled to unit length, largest-
  // magnitude entry positive (the first such entry on ties)
  for (int j = 0; j < R; ++j) {
    const int col = order[j] & (D - 1);
    float* dstj = basis + ((size_t)row * R + j) * D;
    if (tid < 64) {
      float best = -1.f;
      int bidx = 0;
      for (int e = tid; e < D; e += 64) {
        const float a = fabsf(V[e][col]);
        if (a > best) { best = a; bidx = e; }
      }
      // wave argmax, first index on ties
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const float ob = __shfl_xor(best, off);
        const int oi = __shfl_xor(bidx, off);
        if (ob > best || (ob == best && oi < bidx)) { best = ob; bidx = oi; }
      }
      // unit length (the accumulated rotations drift by ~1e-5 at d = 128)
      float ss = 0.f;
      for (int e = tid; e < D; e += 64) ss += V[e][col] * V[e][col];
      ss = wave_sum_f32(ss);
      const float sgn = (V[bidx][col] < 0.f ? -1.f : 1.f) / sqrtf(ss);
      for (int e = tid; e < D; e += 64) dstj[e] = sgn * V[e][col];
    }
  }
}

template <int D, int PS, bool F16>
__global__ __launch_bounds__(64) void summary_basis_kernel(
    const uint16_t* __restrict__ k16, const int32_t* __restrict__ block_table, int max_pages,
    const int32_t* __restrict__ entries, const int32_t* __restrict__ n_valid, int Hkv, int R,
    const float* __restrict__ basis, uint16_t* __restrict__ mu_out, float* __restrict__ lam_out,
    float* __restrict__ log_n) {
  constexpr int CPL = D / 64;   // columns per lane
  __shared__ float X[PS][D + 1];
  __shared__ float U[8][D];

  const int lane = threadIdx.x;
  const int i = blockIdx.x / Hkv, g = blockIdx.x - (blockIdx.x / Hkv) * Hkv;
  const int sb = entries[2 * i], sp = entries[2 * i + 1];   // sequence, logical page
  const int phys = block_table[(size_t)sb * max_pages + sp];
  int nv = n_valid[i];
  nv = nv < 0 ? 0 : (nv > PS ? PS : nv);
  const uint16_t* src = k16 + ((size_t)phys * Hkv + g) * PS * D;
  const size_t rec = ((size_t)sb * Hkv + g) * max_pages + sp;
  uint16_t* mdst = mu_out + rec * D;
  float* ldst = lam_out + rec * R;
  float* ln = log_n + (size_t)sb * max_pages + sp;

  if (nv == 0) {
    for (int e = lane; e < D; e += 64) mdst[e] = 0;
    if (lane < R) ldst[lane] = 0.f;
    if (g == 0 && lane == 0) *ln = -INFINITY;
    return;
  }
  const float* ub = basis + ((size_t)sb * Hkv + g) * R * D;
  for (int idx = lane; idx < R * D; idx += 64) U[idx / D][idx - (idx / D) * D] = ub[idx];
  // mean (token order, float32) and centred keys
#pragma unroll
  for (int c = 0; c < CPL; ++c) {
    const int e = lane + 64 * c;
    float s = 0.f;
    for (int t = 0; t < nv; ++t) s += h16_to_f32<F16>(src[(size_t)t * D + e]);
    const float mu = s / (float)nv;
    mdst[e] = (uint16_t)f32_to_bf16_rne(mu);
    for (int t = 0; t < PS; ++t)
      X[t][e] = t < nv ? h16_to_f32<F16>(src[(size_t)t * D + e]) - mu : 0.f;
  }
  __syncthreads();
  // lam_j = mean over valid tokens of the squared projection on u_j
  const float inv_n = 1.f / (float)nv;
  for (int j = 0; j < R; ++j) {
    float sq = 0.f;
    for (int t = lane; t < nv; t += 64) {
      float pj = 0.f;
      for (int e = 0; e < D; ++e) pj = __builtin_fmaf(U[j][e], X[t][e], pj);
      sq += pj * pj;
    }
    const float tot = wave_sum_f32(sq);
    if (lane == 0) ldst[j] = tot * inv_n;
  }
  if (g == 0 && lane == 0) *ln = logf((float)nv);
}

hipError_t launch_basis_build(const kv_layout& L, const void* k16, const int32_t* block_table,
                              const int32_t* seq_lens, int B, int max_pages, float* basis, float* mean,
                              float* part, hipStream_t st) {
  const int rows = B * L.num_kv_heads;
  const int n_chunks = basis_chunks(max_pages);
  const dim3 gc(n_chunks, rows);
  const bool f16 = L.kv_dtype == KV_F16;
  const uint16_t* k = (const uint16_t*)k16;
#define KVS_COV(D_, F_) hipLaunchKernelGGL((basis_cov_kernel<D_, F_>), gc, dim3((D_ / 8) * (D_ / 8)), 0, st, k, \
                                           block_table, seq_lens, L.num_kv_heads, L.page_size, max_pages, \
                                           kBasisChunkPages, n_chunks, part)
  if (L.head_dim == 64) { if (f16) KVS_COV(64, true); else KVS_COV(64, false); }
  else { if (f16) KVS_COV(128, true); else KVS_COV(128, false); }
#undef KVS_COV
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  if (L.head_dim == 64)
    hipLaunchKernelGGL((basis_eigen_kernel<64>), dim3(rows), dim3(64), 0, st, part, n_chunks, L.rank, basis, mean);
  else
    hipLaunchKernelGGL((basis_eigen_kernel<128>), dim3(rows), dim3(256), 0, st, part, n_chunks, L.rank, basis, mean);
  return hipGetLastError();
}

hipError_t launch_summary_build_basis(const kv_layout& L, const void* k16, const int32_t* block_table,
                                      int max_pages, const int32_t* entries, const int32_t* n_valid, int n,
                                      const float* basis, void* mu, float* lam, float* log_n,
                                      hipStream_t st) {
  const dim3 grid(n * L.num_kv_heads);
  const bool f16 = L.kv_dtype == KV_F16;
  const uint16_t* k = (const uint16_t*)k16;
  uint16_t* m = (uint16_t*)mu;
#define KVS_SBB(D_, PS_, F_) hipLaunchKernelGGL((summary_basis_kernel<D_, PS_, F_>), grid, dim3(64), 0, st, \
                                                k, block_table, max_pages, entries, n_valid, L.num_kv_heads, \
                                                L.rank, basis, m, lam, log_n)
  if (L.head_dim == 64) {
    if (L.page_size == 16) { if (f16) KVS_SBB(64, 16, true); else KVS_SBB(64, 16, false); }
    else { if (f16) KVS_SBB(64, 32, true); else KVS_SBB(64, 32, false); }
  } else {
    if (L.page_size == 16) { if (f16) KVS_SBB(128, 16, true); else KVS_SBB(128, 16, false); }
    else { if (f16) KVS_SBB(128, 32, true); else KVS_SBB(128, 32, false); }
  }
#undef KVS_SBB
  return hipGetLastError();
}

}  // namespace kvs
