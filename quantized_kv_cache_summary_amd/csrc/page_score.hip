// Quad page score: for every logical page of a (sequence, KV head) row and
// every query head of its group,
//   s = log n + tau q.mu + (tau^2 / 2) sum_j (q.w_j)^2
// AMASS (amass-kv 0.1.1 project page), "What is in the box" item 1 (quadratic
// Gaussian-MGF score from a tiny per-page summary) and "Benchmarking" (the
// score stage is bandwidth-bound and measured against the HBM roofline).
//
// gfx950 design.  The step is a stream over the summary records (HBM-bound);
// each wave scores one 16-page tile (score_tile.h: one MFMA per 32 head-dim
// elements of 16 query heads against 16 record vectors).  A wave issues all
// of its tile's record loads before its first MFMA, so it waits on memory
// once and a CU keeps a few hundred KB in flight.  Each block covers 64 pages
// of one row and also emits the (max, sum exp) of its pages per head, so the
// selector never re-reads all scores to normalise.

#include "device.h"
#include "launch.h"
#include "score_tile.h"

namespace kvs {

constexpr int kScoreWaves = kScorePagesPerBlock / 16;   // one 16-page tile per wave

template <int D, int R, bool F16>
__global__ __launch_bounds__(64 * kScoreWaves) void page_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ summary,
    const float* __restrict__ log_n, const int32_t* __restrict__ seq_lens, int Hkv, int G, int P,
    int max_pages, int n_tiles, float tau, float* __restrict__ head_scores,
    float* __restrict__ lse_partial) {
  const int row = blockIdx.y;
  const int b = row / Hkv;
  const int g = row - b * Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)

  const int L = seq_lens[b];
  int Np = L > 0 ? (L + P - 1) / P : 0;
  Np = Np < max_pages ? Np : max_pages;
  const int base = blockIdx.x * kScorePagesPerBlock + wave * 16;

  ScoreTile<D, R, F16> t;
  score_tile_issue<D, R, F16>(t, q, summary, log_n, b, g, Hkv, G, max_pages, base);
  __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the first MFMA
  float run_m, run_s;
  score_tile_finish<D, R, F16, false>(t, row, G, Np, max_pages, base, tau, head_scores, run_m, run_s);

  // combine the waves in a fixed order
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
                                 const float* log_n, const int32_t* sl, int B,
                                 int max_pages, float tau, float* hs, float* lp, hipStream_t st) {
  const int G = L.num_q_heads / L.num_kv_heads;
  const int n_tiles = score_tiles(max_pages);
  dim3 grid(n_tiles, B * L.num_kv_heads);
  hipLaunchKernelGGL((page_score_kernel<D, R, F16>), grid, dim3(64 * kScoreWaves), 0, st,
                     (const uint16_t*)q, (const uint16_t*)summary, log_n, sl, L.num_kv_heads, G,
                     L.page_size, max_pages, n_tiles, tau, hs, lp);
  return hipGetLastError();
}

template <int D, bool F16>
static hipError_t launch_score_r(const kv_layout& L, const void* q, const void* summary,
                                 const float* log_n, const int32_t* sl, int B,
                                 int max_pages, float tau, float* hs, float* lp, hipStream_t st) {
  switch (L.rank) {
    case 1: return launch_score_t<D, 1, F16>(L, q, summary, log_n, sl, B, max_pages, tau, hs, lp, st);
    case 2: return launch_score_t<D, 2, F16>(L, q, summary, log_n, sl, B, max_pages, tau, hs, lp, st);
    case 4: return launch_score_t<D, 4, F16>(L, q, summary, log_n, sl, B, max_pages, tau, hs, lp, st);
    default: return launch_score_t<D, 8, F16>(L, q, summary, log_n, sl, B, max_pages, tau, hs, lp, st);
  }
}

hipError_t launch_page_score(const kv_layout& L, const void* q, const void* summary,
                             const float* log_n, const int32_t* seq_lens,
                             int B, int max_pages, float tau, float* head_scores, float* lse_partial,
                             hipStream_t st) {
  const bool f16 = L.kv_dtype == KV_F16;
  if (L.head_dim == 64)
    return f16 ? launch_score_r<64, true>(L, q, summary, log_n, seq_lens, B, max_pages, tau, head_scores, lse_partial, st)
               : launch_score_r<64, false>(L, q, summary, log_n, seq_lens, B, max_pages, tau, head_scores, lse_partial, st);
  return f16 ? launch_score_r<128, true>(L, q, summary, log_n, seq_lens, B, max_pages, tau, head_scores, lse_partial, st)
             : launch_score_r<128, false>(L, q, summary, log_n, seq_lens, B, max_pages, tau, head_scores, lse_partial, st);
}

}  // namespace kvs
