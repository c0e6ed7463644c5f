// r8 low-rank page score.  AMASS (amass-kv 0.1.1 project page), "Quickstart"
// (the r8 low-rank fallback score) and "Headline results" (r8 keeps per-key
// low-rank state, which quad drops).  Every key keeps its coordinates in the
// row's shared basis about the row mean,
//   c_tj = bfloat16( u_j . (k_t - m) ),
// and a page scores as the log-mass of its approximated keys,
//   s_p = tau q.m + log sum_{t in p} exp( tau sum_j (q.u_j) c_tj ).
//
// Score kernel: a block covers 64 pages of one row (the quad score's tiles,
// so the selector reads the same partials).  The block first forms
// tau q_h.u_j and tau q_h.m for its heads from the query, row basis and mean
// staged in LDS (one wave per product, lanes over the head dim).  Then each
// wave takes 16 pages, four lanes per page, each lane P/4 consecutive tokens
// whose coordinates are contiguous (a wave reads 16 whole pages, one
// contiguous span); the four lanes share the page's maximum and sum their
// exponentials through DPP quad permutes, and the per-head tile partials are
// DPP wave reductions.

#include "device.h"
#include "launch.h"

namespace kvs {

constexpr int kLrTiles = 4;                                   // score tiles per block
constexpr int kLrPages = kLrTiles * kScorePagesPerBlock;     // pages per block
constexpr int kLrWaves = kLrPages / 16;
constexpr int kLrTileWaves = kScorePagesPerBlock / 16;   // waves per score tile

// lane exchanges within groups of four lanes (DPP quad permutes, no LDS)
__device__ __forceinline__ float quad_xor1(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0xB1, 0xF, 0xF, false));   // [1,0,3,2]
}
__device__ __forceinline__ float quad_xor2(float x) {
  return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(x), 0x4E, 0xF, 0xF, false));   // [2,3,0,1]
}

// coordinates of appended pages: one 64-thread block per (entry, KV head)
template <int D, int R, bool F16>
__global__ __launch_bounds__(64) void lowrank_coords_kernel(const uint16_t* __restrict__ k16,
                                                            const int32_t* __restrict__ block_table, int Hkv,
                                                            int P, int max_pages, const int32_t* __restrict__ entries,
                                                            const int32_t* __restrict__ n_valid,
                                                            const float* __restrict__ basis,
                                                            const float* __restrict__ mean,
                                                            uint16_t* __restrict__ coords) {
  __shared__ float sm[D];
  __shared__ float su[R][D];
  const int i = blockIdx.x, g = blockIdx.y, tid = threadIdx.x;
  const int b = entries[2 * i], p = entries[2 * i + 1];
  const int row = b * Hkv + g;
  for (int e = tid; e < D; e += 64) sm[e] = mean[(size_t)row * D + e];
  for (int e = tid; e < R * D; e += 64) su[e / D][e % D] = basis[(size_t)row * R * D + e];
  __syncthreads();
  int n = n_valid[i];
  n = n < 0 ? 0 : (n > P ? P : n);
  const int phys = block_table[(size_t)b * max_pages + p];
  const uint16_t* kp = k16 + ((size_t)phys * Hkv + g) * P * D;
  uint16_t* dst = coords + (((size_t)row * max_pages + p) * P) * R;
  for (int o = tid; o < P * R; o += 64) {
    const int t = o / R, j = o - t * R;
    float c = 0.f;
    if (t < n) {
      const uint16_t* kt = kp + (size_t)t * D;
      for (int e = 0; e < D; e += 8) {
        const u32x4_t w = ld16(kt + e);
#pragma unroll
        for (int h = 0; h < 4; ++h) {
          c = __builtin_fmaf(lo16<F16>(w[h]) - sm[e + 2 * h], su[j][e + 2 * h], c);
          c = __builtin_fmaf(hi16<F16>(w[h]) - sm[e + 2 * h + 1], su[j][e + 2 * h + 1], c);
        }
      }
    }
    dst[o] = (uint16_t)f32_to_bf16_rne(c);
  }
}

template <int D, int R, int GM, bool F16>
__global__ __launch_bounds__(64 * kLrWaves) void page_score_lowrank_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ coords, const float* __restrict__ mean,
    const float* __restrict__ basis, const int32_t* __restrict__ seq_lens, int Hkv, int G, int P, int max_pages,
    int n_tiles, float tau, float* __restrict__ head_scores, float* __restrict__ lse_partial) {
  constexpr int NT = 64 * kLrWaves;
  __shared__ float sv[R + 1][D];          // basis rows, then the mean
  __shared__ float qv[GM][R + 1];         // tau q_h.u_j, then tau q_h.m
  __shared__ float red_m[kLrWaves][GM], red_s[kLrWaves][GM];
  const int row = blockIdx.y, b = row / Hkv, g = row - b * Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // page data first: its loads are in flight while the projections are formed
  const int pw = lane >> 2, quarter = lane & 3;
  const int tpl = P / 4;                  // tokens per lane (4 or 8)
  const int p = blockIdx.x * kLrPages + wave * 16 + pw;
  const int pc = p < max_pages ? p : max_pages - 1;
  const uint16_t* cp = coords + (((size_t)row * max_pages + pc) * P + quarter * tpl) * R;
  // a token's R bfloat16 coordinates are one aligned load (16, 8, 4 or 2 bytes)
  constexpr int CW = (R + 1) / 2;         // 32-bit words per token
  uint32_t cw[8][CW];
#pragma unroll
  for (int t = 0; t < 8; ++t) {
    if (t >= tpl) continue;
    const uint16_t* ct = cp + t * R;
    if constexpr (R == 8) {
      const u32x4_t w = ld16(ct);
#pragma unroll
      for (int k = 0; k < 4; ++k) cw[t][k] = w[k];
    } else if constexpr (R == 4) {
      const u32x2_t w = *reinterpret_cast<const u32x2_t*>(ct);
      cw[t][0] = w[0];
      cw[t][1] = w[1];
    } else if constexpr (R == 2) {
      cw[t][0] = *reinterpret_cast<const uint32_t*>(ct);
    } else {
      cw[t][0] = *ct;
    }
  }

  __shared__ float sq[GM][D];              // the group's query heads
  const int Hq = Hkv * G;
  // every staging load is requested before any is stored
  constexpr int NSV = ((R + 1) * D + NT - 1) / NT, NSQ = (GM * D + NT - 1) / NT;
  float tv[NSV];
  uint16_t tq[NSQ];
#pragma unroll
  for (int i = 0; i < NSV; ++i) {
    const int e = tid + i * NT, j = e / D, x = e - j * D;
    tv[i] = e >= (R + 1) * D ? 0.f : (j < R ? basis[((size_t)row * R + j) * D + x] : mean[(size_t)row * D + x]);
  }
#pragma unroll
  for (int i = 0; i < NSQ; ++i) {
    const int e = tid + i * NT, h = e / D, x = e - h * D;
    tq[i] = h < G ? q[((size_t)b * Hq + (size_t)g * G + h) * D + x] : (uint16_t)0;
  }
#pragma unroll
  for (int i = 0; i < NSV; ++i) {
    const int e = tid + i * NT;
    if (e < (R + 1) * D) sv[e / D][e % D] = tv[i];
  }
#pragma unroll
  for (int i = 0; i < NSQ; ++i) {
    const int e = tid + i * NT;
    if (e / D < G) sq[e / D][e % D] = h16_to_f32<F16>(tq[i]);
  }
  __syncthreads();
  // tau q_h.u_j and tau q_h.m: one wave per product, lanes over the head dim
  for (int o = wave; o < G * (R + 1); o += kLrWaves) {
    const int h = o / (R + 1), j = o - h * (R + 1);
    float part = 0.f;
#pragma unroll
    for (int e = lane; e < D; e += 64) part = __builtin_fmaf(sq[h][e], sv[j][e], part);
    part = wave_sum_f32(part);
    if (lane == 0) qv[h][j] = tau * part;
  }
  __syncthreads();

  const int L = seq_lens[b];
  int Np = L > 0 ? (L + P - 1) / P : 0;
  Np = Np < max_pages ? Np : max_pages;
  int n = p < Np ? L - p * P : 0;
  n = n > P ? P : n;
  float sc[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    sc[h] = -INFINITY;
    if (h >= G) continue;
    float z[8];
    float zm = -INFINITY;
#pragma unroll
    for (int t = 0; t < 8; ++t) {
      z[t] = -INFINITY;
      if (t < tpl && quarter * tpl + t < n) {
        float a = 0.f;
#pragma unroll
        for (int j = 0; j < R; ++j) {
          const uint32_t wj = cw[t][j >> 1];
          a = __builtin_fmaf(qv[h][j], __uint_as_float((j & 1) ? (wj & 0xFFFF0000u) : (wj << 16)), a);
        }
        z[t] = a;
        zm = fmaxf(zm, a);
      }
    }
    // the page's four lanes share one maximum, then sum their exponentials
    zm = fmaxf(zm, quad_xor1(zm));
    zm = fmaxf(zm, quad_xor2(zm));
    float zs = 0.f;
    if (zm != -INFINITY) {
#pragma unroll
      for (int t = 0; t < 8; ++t)
        if (t < tpl && z[t] != -INFINITY) zs += __expf(z[t] - zm);
    }
    zs += quad_xor1(zs);
    zs += quad_xor2(zs);
    sc[h] = zm == -INFINITY ? -INFINITY : qv[h][R] + zm + __logf(zs);
    if (quarter == (h & 3) && p < max_pages) head_scores[((size_t)row * G + h) * max_pages + p] = sc[h];
  }
  // per head (max, sum exp) over the block's pages: the wave's 16 pages (one
  // lane of each), then the waves in order
#pragma unroll
  for (int h = 0; h < GM; ++h) {
    if (h >= G) continue;
    const float M = wave_max_f32(sc[h]);
    const float S = wave_sum_f32(quarter == 0 && sc[h] != -INFINITY ? __expf(sc[h] - M) : 0.f);
    if (lane == 0) { red_m[wave][h] = M; red_s[wave][h] = S; }
  }
  __syncthreads();
  // one partial per 64-page score tile: waves [tile * kLrTileWaves, +kLrTileWaves)
  if (tid < kLrTiles * G) {
    const int h = tid % G, part = tid / G;
    const int tile = blockIdx.x * kLrTiles + part;
    const int w0 = part * kLrTileWaves;
    float m = red_m[w0][h], s = red_s[w0][h];
#pragma unroll
    for (int w = 1; w < kLrTileWaves; ++w) lse_merge(m, s, red_m[w0 + w][h], red_s[w0 + w][h]);
    if (tile < n_tiles) {
      float* dst = lse_partial + (((size_t)row * n_tiles + tile) * G + h) * 2;
      dst[0] = m;
      dst[1] = s;
    }
  }
}

template <int D, int R, bool F16>
static hipError_t launch_lr_score(const kv_layout& L, const void* q, const void* coords, const float* mean,
                                  const float* basis, const int32_t* sl, int B, int max_pages, float tau,
                                  float* hs, float* lp, hipStream_t st) {
  const int G = L.num_q_heads / L.num_kv_heads;
  const int n_tiles = score_tiles(max_pages);
  const dim3 grid((n_tiles + kLrTiles - 1) / kLrTiles, B * L.num_kv_heads);
#define KVS_LR(GM_) hipLaunchKernelGGL((page_score_lowrank_kernel<D, R, GM_, F16>), grid, dim3(64 * kLrWaves), 0, st, \
                       (const uint16_t*)q, (const uint16_t*)coords, mean, basis, sl, L.num_kv_heads, G, L.page_size,   \
                       max_pages, n_tiles, tau, hs, lp)
  if (G <= 4) KVS_LR(4);
  else if (G <= 8) KVS_LR(8);
  else KVS_LR(16);
#undef KVS_LR
  return hipGetLastError();
}

template <int D, bool F16>
static hipError_t launch_lr_score_r(const kv_layout& L, const void* q, const void* coords, const float* mean,
                                    const float* basis, const int32_t* sl, int B, int max_pages, float tau,
                                    float* hs, float* lp, hipStream_t st) {
  switch (L.rank) {
    case 1: return launch_lr_score<D, 1, F16>(L, q, coords, mean, basis, sl, B, max_pages, tau, hs, lp, st);
    case 2: return launch_lr_score<D, 2, F16>(L, q, coords, mean, basis, sl, B, max_pages, tau, hs, lp, st);
    case 4: return launch_lr_score<D, 4, F16>(L, q, coords, mean, basis, sl, B, max_pages, tau, hs, lp, st);
    default: return launch_lr_score<D, 8, F16>(L, q, coords, mean, basis, sl, B, max_pages, tau, hs, lp, st);
  }
}

hipError_t launch_page_score_lowrank(const kv_layout& L, const void* q, const void* coords, const float* mean,
                                     const float* basis, const int32_t* seq_lens, int B, int max_pages,
                                     float tau, float* head_scores, float* lse_partial, hipStream_t st) {
  const bool f16 = L.kv_dtype == KV_F16;
  if (L.head_dim == 64)
    return f16 ? launch_lr_score_r<64, true>(L, q, coords, mean, basis, seq_lens, B, max_pages, tau, head_scores, lse_partial, st)
               : launch_lr_score_r<64, false>(L, q, coords, mean, basis, seq_lens, B, max_pages, tau, head_scores, lse_partial, st);
  return f16 ? launch_lr_score_r<128, true>(L, q, coords, mean, basis, seq_lens, B, max_pages, tau, head_scores, lse_partial, st)
             : launch_lr_score_r<128, false>(L, q, coords, mean, basis, seq_lens, B, max_pages, tau, head_scores, lse_partial, st);
}

template <int D, int R, bool F16>
static hipError_t launch_lr_coords(const kv_layout& L, const void* k16, const int32_t* bt, int max_pages,
                                   const int32_t* entries, const int32_t* n_valid, int n, const float* basis,
                                   const float* mean, void* coords, hipStream_t st) {
  hipLaunchKernelGGL((lowrank_coords_kernel<D, R, F16>), dim3(n, L.num_kv_heads), dim3(64), 0, st,
                     (const uint16_t*)k16, bt, L.num_kv_heads, L.page_size, max_pages, entries, n_valid, basis, mean,
                     (uint16_t*)coords);
  return hipGetLastError();
}

template <int D, bool F16>
static hipError_t launch_lr_coords_r(const kv_layout& L, const void* k16, const int32_t* bt, int max_pages,
                                     const int32_t* entries, const int32_t* n_valid, int n, const float* basis,
                                     const float* mean, void* coords, hipStream_t st) {
  switch (L.rank) {
    case 1: return launch_lr_coords<D, 1, F16>(L, k16, bt, max_pages, entries, n_valid, n, basis, mean, coords, st);
    case 2: return launch_lr_coords<D, 2, F16>(L, k16, bt, max_pages, entries, n_valid, n, basis, mean, coords, st);
    case 4: return launch_lr_coords<D, 4, F16>(L, k16, bt, max_pages, entries, n_valid, n, basis, mean, coords, st);
    default: return launch_lr_coords<D, 8, F16>(L, k16, bt, max_pages, entries, n_valid, n, basis, mean, coords, st);
  }
}

hipError_t launch_lowrank_coords(const kv_layout& L, const void* k16, const int32_t* block_table, int max_pages,
                                 const int32_t* entries, const int32_t* n_valid, int n, const float* basis,
                                 const float* mean, void* coords, hipStream_t st) {
  const bool f16 = L.kv_dtype == KV_F16;
  if (L.head_dim == 64)
    return f16 ? launch_lr_coords_r<64, true>(L, k16, block_table, max_pages, entries, n_valid, n, basis, mean, coords, st)
               : launch_lr_coords_r<64, false>(L, k16, block_table, max_pages, entries, n_valid, n, basis, mean, coords, st);
  return f16 ? launch_lr_coords_r<128, true>(L, k16, block_table, max_pages, entries, n_valid, n, basis, mean, coords, st)
             : launch_lr_coords_r<128, false>(L, k16, block_table, max_pages, entries, n_valid, n, basis, mean, coords, st);
}

}  // namespace kvs
