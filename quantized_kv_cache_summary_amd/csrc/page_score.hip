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
// loads and finishes scores.  Summaries are stored in logical page order per
// (sequence, KV head), so a row's records are one contiguous stream and no
// block-table lookup precedes the loads.  Record vectors are the MFMA A rows;
// a load instruction reads 64 contiguous bytes of each of 16 vectors.  Rows
// are assigned so that every lane ends
// with all quantities of its own pages in its own accumulator registers:
//   mean tile: A row r = 4g'+i holds mu of page 4i + g'
//   direction tiles: the R w's of page 4m + g' sit in rows of lane group g'
// (the MFMA writes rows 4g'..4g'+3 to lane group g').  No cross-lane
// reduction is needed per page.  A wave owns one 16-page tile and issues all
// of the tile's record loads before its first MFMA, so each wave waits on
// memory once and a CU keeps a few hundred KB in flight.  Each block covers
// 64 pages of one row and also emits the (max, sum exp) of its pages per
// head, so the selector never re-reads all scores to normalise.

#include "device.h"
#include "launch.h"

namespace kvs {

constexpr int kScoreWaves = kScorePagesPerBlock / 16;   // one 16-page tile per wave

template <int D, int R, bool F16>
__global__ __launch_bounds__(64 * kScoreWaves) void page_score_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ summary,
    const float* __restrict__ log_n, const int32_t* __restrict__ seq_lens, int Hkv, int G, int P,
    int max_pages, int n_tiles, float tau, float* __restrict__ head_scores,
    float* __restrict__ lse_partial) {
  constexpr int KS = D / 32;          // MFMA k-steps per vector
  constexpr int REC = (1 + R) * D;    // record length (elements)
  constexpr int PPL = (R <= 4) ? 4 / R : 1;   // pages per lane group in one direction tile

  const int row = blockIdx.y;
  const int b = row / Hkv;
  const int g = row - b * Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int col = lane & 15;   // A row within the tile; also the output column (= head)
  const int kg = lane >> 4;    // A k-group; also the output row group

  const int L = seq_lens[b];
  int Np = L > 0 ? (L + P - 1) / P : 0;
  Np = Np < max_pages ? Np : max_pages;
  const int base = blockIdx.x * kScorePagesPerBlock + wave * 16;
  // pages past the end are read from a clamped, always allocated record and
  // their results dropped, so every load below is unconditional
  auto clampp = [&](int p) { return p < max_pages ? p : max_pages - 1; };

  float ln[4];
#pragma unroll
  for (int m = 0; m < 4; ++m) ln[m] = log_n[(size_t)b * max_pages + clampp(base + 4 * m + kg)];

  // Element assignment: at k-step s, k-group kg holds head-dim elements
  // [32s + 8kg, 32s + 8kg + 8), so one load instruction reads 64 contiguous
  // bytes of each of 16 vectors.  The query uses the same assignment.
  u32x4_t qh[KS], ql[KS];
  {
    const int Hq = Hkv * G;
    const uint32_t keep = col < G ? 0xFFFFFFFFu : 0u;
    const uint16_t* qp = q + ((size_t)b * Hq + (size_t)g * G + (col < G ? col : 0)) * D + 8 * kg;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t raw = ld16(qp + 32 * s);
#pragma unroll
      for (int w = 0; w < 4; ++w) raw[w] &= keep;
      if constexpr (!F16) {
        qh[s] = raw;
      } else {
        // a float16 query is split exactly into two bfloat16 halves (11 = 8 + 3
        // bits) because the summary is bfloat16
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

  // Every record vector this lane feeds to the MFMA, loaded before any math.
  //   mean tile: A row r = col holds page (r & 3) * 4 + (r >> 2)
  //   direction tile wt: A row r holds w_j of page pl (mapping below)
  const uint16_t* rowrec = summary + (size_t)row * max_pages * REC + 8 * kg;
  u32x4_t a[1 + R][KS];
  {
    const uint16_t* src = rowrec + (size_t)clampp(base + (col & 3) * 4 + (col >> 2)) * REC;
#pragma unroll
    for (int s = 0; s < KS; ++s) a[0][s] = ld16(src + 32 * s);
  }
#pragma unroll
  for (int wt = 0; wt < R; ++wt) {
    const int gq = col >> 2, i = col & 3;
    int pl, j;
    if constexpr (R <= 4) { pl = 4 * (wt * PPL + i / R) + gq; j = i % R; }
    else { pl = 4 * (wt / 2) + gq; j = 4 * (wt % 2) + i; }
    const uint16_t* src = rowrec + (size_t)clampp(base + pl) * REC + (size_t)(1 + j) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) a[1 + wt][s] = ld16(src + 32 * s);
  }

  __builtin_amdgcn_sched_barrier(0);   // every load above is issued before the first MFMA

  f32x4_t acc_mu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    acc_mu = mfma16<false>(a[0][s], qh[s], acc_mu);
    if constexpr (F16) acc_mu = mfma16<false>(a[0][s], ql[s], acc_mu);
  }
  float quad[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int wt = 0; wt < R; ++wt) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      acc = mfma16<false>(a[1 + wt][s], qh[s], acc);
      if constexpr (F16) acc = mfma16<false>(a[1 + wt][s], ql[s], acc);
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int m = (R <= 4) ? wt * PPL + ii / R : wt / 2;
      quad[m] += acc[ii] * acc[ii];
    }
  }

  // scores of pages base + 4m + kg for head col
  const float c1 = tau, c2 = 0.5f * tau * tau;
  float run_m = -INFINITY, run_s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int p = base + 4 * m + kg;
    const float s = p < Np ? ln[m] + c1 * acc_mu[m] + c2 * quad[m] : -INFINITY;
    if (col < G && p < max_pages) head_scores[((size_t)row * G + col) * max_pages + p] = s;
    if (p < Np && s != -INFINITY) lse_merge(run_m, run_s, s, 1.f);
  }

  // combine the four lane groups (same head), then the waves, in a fixed order
  {
    float m2 = __shfl_xor(run_m, 16), s2 = __shfl_xor(run_s, 16);
    lse_merge(run_m, run_s, m2, s2);
    m2 = __shfl_xor(run_m, 32);
    s2 = __shfl_xor(run_s, 32);
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
