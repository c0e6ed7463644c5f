// Quad page score: for every logical page of a (sequence, KV head) row and
// every query head of its group,
//   s = log n + tau q.mu + (tau^2 / 2) sum_j (q.w_j)^2
// AMASS (amass-kv 0.1.1 project page), "What is in the box" item 1 (quadratic
// Gaussian-MGF score from a tiny per-page summary) and "Benchmarking" (the
// score stage is bandwidth-bound and measured against the HBM roofline).
//
// gfx950 design.  The step is a stream over the summary records (HBM-bound).
// The dot products q.mu and q.w_j of 16 query-head columns against 16 summary
// vectors are one 16x16x32 MFMA per 32 head-dim elements, so the VALU only
// loads and finishes scores.  Record vectors are the MFMA A rows; each lane
// loads d/4 contiguous elements (64 bytes at d=128) of one vector, so a wave
// reads whole 256-byte vectors.  Rows are assigned so that every lane ends
// with all quantities of its own pages in its own accumulator registers:
//   mean tile: A row r = 4g'+i holds mu of page 4i + g'
//   direction tiles: the R w's of page 4m + g' sit in rows of lane group g'
// (the MFMA writes rows 4g'..4g'+3 to lane group g').  No cross-lane
// reduction is needed per page.  Each block covers 128 pages of one row
// (4 waves x 2 tiles x 16 pages) and also emits the (max, sum exp) of its
// pages per head, so the selector never re-reads all scores to normalise.

#include "device.h"
#include "launch.h"

namespace kvs {

constexpr int kScoreWaves = 4;
constexpr int kScoreTilesPerWave = kScorePagesPerBlock / (kScoreWaves * 16);

template <int D, int R, bool F16>
__global__ __launch_bounds__(256) void page_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ summary,
    const float* __restrict__ log_n, const int32_t* __restrict__ block_table,
    const int32_t* __restrict__ seq_lens, int Hkv, int G, int P, int max_pages, int n_tiles,
    float tau, float* __restrict__ head_scores, float* __restrict__ lse_partial) {
  constexpr int KS = D / 32;          // MFMA k-steps per vector
  constexpr int EPL = D / 4;          // vector elements held by one lane
  constexpr int REC = (1 + R) * D;    // record length (elements)
  constexpr int PPL = (R <= 4) ? 4 / R : 1;   // pages per lane group in one direction tile

  const int row = blockIdx.y;
  const int b = row / Hkv;
  const int g = row - b * Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = threadIdx.x >> 6;
  const int col = lane & 15;   // A row within a tile; also the output column (= head)
  const int kg = lane >> 4;    // A k-group; also the output row group

  const int L = seq_lens[b];
  int Np = L > 0 ? (L + P - 1) / P : 0;
  Np = Np < max_pages ? Np : max_pages;

  // B operand: query head `col` (zero beyond G), elements kg*EPL + 8s + [0, 8).
  // A float16 query is split exactly into two bfloat16 halves (11 = 8 + 3 bits)
  // because the summary is bfloat16.
  u32x4_t qh[KS], ql[KS];
  {
    const int Hq = Hkv * G;
    const uint16_t* qp = q + ((size_t)b * Hq + (size_t)g * G + (col < G ? col : 0)) * D + kg * EPL;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t raw = col < G ? ld16(qp + 8 * s) : u32x4_t{0, 0, 0, 0};
      if constexpr (!F16) {
        qh[s] = raw;
      } else {
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float f0 = f16_bits_to_f32(raw[w] & 0xFFFFu), f1 = f16_bits_to_f32(raw[w] >> 16);
          const uint32_t h0 = __float_as_uint(f0) & 0xFFFF0000u, h1 = __float_as_uint(f1) & 0xFFFF0000u;
          const uint32_t l0 = __float_as_uint(f0 - __uint_as_float(h0)) >> 16;
          const uint32_t l1 = __float_as_uint(f1 - __uint_as_float(h1)) >> 16;
          qh[s][w] = (h0 >> 16) | h1;
          ql[s][w] = l0 | (l1 << 16);
        }
      }
    }
  }

  const int32_t* bt = block_table + (size_t)b * max_pages;
  const size_t rec_g = (size_t)g * REC + (size_t)kg * EPL;
  const float c1 = tau, c2 = 0.5f * tau * tau;
  float run_m = -INFINITY, run_s = 0.f;

  const int page0 = blockIdx.x * kScorePagesPerBlock + wave * (kScoreTilesPerWave * 16);
#pragma unroll
  for (int t = 0; t < kScoreTilesPerWave; ++t) {
    const int base = page0 + t * 16;
    if (base >= max_pages) break;

    // mean tile
    f32x4_t acc_mu = {0.f, 0.f, 0.f, 0.f};
    {
      const int p = base + (col & 3) * 4 + (col >> 2);
      u32x4_t a[KS];
      if (p < Np) {
        const uint16_t* src = summary + (size_t)bt[p] * Hkv * REC + rec_g;
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = ld16(src + 8 * s);
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = u32x4_t{0, 0, 0, 0};
      }
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        acc_mu = mfma16<false>(a[s], qh[s], acc_mu);
        if constexpr (F16) acc_mu = mfma16<false>(a[s], ql[s], acc_mu);
      }
    }

    // direction tiles
    float quad[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int wt = 0; wt < R; ++wt) {
      const int gq = col >> 2, i = col & 3;
      int pl, j;
      if constexpr (R <= 4) { pl = 4 * (wt * PPL + i / R) + gq; j = i % R; }
      else { pl = 4 * (wt / 2) + gq; j = 4 * (wt % 2) + i; }
      const int p = base + pl;
      u32x4_t a[KS];
      if (p < Np) {
        const uint16_t* src = summary + (size_t)bt[p] * Hkv * REC + rec_g + (size_t)(1 + j) * D;
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = ld16(src + 8 * s);
      } else {
#pragma unroll
        for (int s = 0; s < KS; ++s) a[s] = u32x4_t{0, 0, 0, 0};
      }
      f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int s = 0; s < KS; ++s) {
        acc = mfma16<false>(a[s], qh[s], acc);
        if constexpr (F16) acc = mfma16<false>(a[s], ql[s], acc);
      }
#pragma unroll
      for (int ii = 0; ii < 4; ++ii) {
        const int m = (R <= 4) ? wt * PPL + ii / R : wt / 2;
        quad[m] += acc[ii] * acc[ii];
      }
    }

    // scores of pages base + 4m + kg for head col
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int p = base + 4 * m + kg;
      float s = -INFINITY;
      if (p < Np) s = log_n[bt[p]] + c1 * acc_mu[m] + c2 * quad[m];
      if (col < G && p < max_pages) head_scores[((size_t)row * G + col) * max_pages + p] = s;
      if (p < Np && s != -INFINITY) lse_merge(run_m, run_s, s, 1.f);
    }
  }

  // combine the four lane groups (same head), then the waves, in a fixed order
  {
    float m2 = __shfl_xor(run_m, 16), s2 = __shfl_xor(run_s, 16);
    if (kg & 1) { float tm = run_m, ts = run_s; run_m = m2; run_s = s2; m2 = tm; s2 = ts; }
    lse_merge(run_m, run_s, m2, s2);
    m2 = __shfl_xor(run_m, 32); s2 = __shfl_xor(run_s, 32);
    if (kg & 2) { float tm = run_m, ts = run_s; run_m = m2; run_s = s2; m2 = tm; s2 = ts; }
    lse_merge(run_m, run_s, m2, s2);
  }
  __shared__ float red_m[kScoreWaves][16], red_s[kScoreWaves][16];
  if (lane < 16) { red_m[wave][lane] = run_m; red_s[wave][lane] = run_s; }
  __syncthreads();
  if (wave == 0 && lane < G) {
    float m = red_m[0][lane], s = red_s[0][lane];
#pragma unroll
    for (int w = 1; w < kScoreWaves; ++w) lse_merge(m, s, red_m[w][lane], red_s[w][lane]);
    float* dst = lse_partial + (((size_t)row * n_tiles + blockIdx.x) * G + lane) * 2;
    dst[0] = m;
    dst[1] = s;
  }
}

template <int D, int R, bool F16>
static hipError_t launch_score_t(const kv_layout& L, const void* q, const void* summary,
                                 const float* log_n, const int32_t* bt, const int32_t* sl, int B,
                                 int max_pages, float tau, float* hs, float* lp, hipStream_t st) {
  const int G = L.num_q_heads / L.num_kv_heads;
  const int n_tiles = score_tiles(max_pages);
  dim3 grid(n_tiles, B * L.num_kv_heads);
  hipLaunchKernelGGL((page_score_kernel<D, R, F16>), grid, dim3(256), 0, st,
                     (const uint16_t*)q, (const uint16_t*)summary, log_n, bt, sl, L.num_kv_heads, G,
                     L.page_size, max_pages, n_tiles, tau, hs, lp);
  return hipGetLastError();
}

template <int D, bool F16>
static hipError_t launch_score_r(const kv_layout& L, const void* q, const void* summary,
                                 const float* log_n, const int32_t* bt, const int32_t* sl, int B,
                                 int max_pages, float tau, float* hs, float* lp, hipStream_t st) {
  switch (L.rank) {
    case 1: return launch_score_t<D, 1, F16>(L, q, summary, log_n, bt, sl, B, max_pages, tau, hs, lp, st);
    case 2: return launch_score_t<D, 2, F16>(L, q, summary, log_n, bt, sl, B, max_pages, tau, hs, lp, st);
    case 4: return launch_score_t<D, 4, F16>(L, q, summary, log_n, bt, sl, B, max_pages, tau, hs, lp, st);
    default: return launch_score_t<D, 8, F16>(L, q, summary, log_n, bt, sl, B, max_pages, tau, hs, lp, st);
  }
}

hipError_t launch_page_score(const kv_layout& L, const void* q, const void* summary,
                             const float* log_n, const int32_t* block_table, const int32_t* seq_lens,
                             int B, int max_pages, float tau, float* head_scores, float* lse_partial,
                             hipStream_t st) {
  const bool f16 = L.kv_dtype == KV_F16;
  if (L.head_dim == 64)
    return f16 ? launch_score_r<64, true>(L, q, summary, log_n, block_table, seq_lens, B, max_pages, tau, head_scores, lse_partial, st)
               : launch_score_r<64, false>(L, q, summary, log_n, block_table, seq_lens, B, max_pages, tau, head_scores, lse_partial, st);
  return f16 ? launch_score_r<128, true>(L, q, summary, log_n, block_table, seq_lens, B, max_pages, tau, head_scores, lse_partial, st)
             : launch_score_r<128, false>(L, q, summary, log_n, block_table, seq_lens, B, max_pages, tau, head_scores, lse_partial, st);
}

}  // namespace kvs
