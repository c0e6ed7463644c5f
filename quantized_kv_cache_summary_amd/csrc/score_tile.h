// One wave's 16-page tile of the quad page score (AMASS, amass-kv 0.1.1
// project page, "What is in the box" item 1: quadratic Gaussian-MGF score from
// a per-page summary):
//   s = log n + tau q.mu + (tau^2 / 2) sum_j (q.w_j)^2
// split into the loads (issue) and the arithmetic (finish), so a kernel can
// request the next tile's records before it finishes the current one.
//
// The dot products q.mu and q.w_j of 16 query-head columns against 16 summary
// vectors are one 16x16x32 MFMA per 32 head-dim elements.  Summaries are in
// logical page order per (sequence, KV head), so a row's records are one
// contiguous stream and no block-table lookup precedes the loads.  Record
// vectors are the MFMA A rows; a load instruction reads 64 contiguous bytes of
// each of 16 vectors.  Rows are assigned so that every lane ends with all
// quantities of its own pages in its own accumulator registers:
//   mean tile: A row r = 4g'+i holds mu of page 4i + g'
//   direction tiles: the R w's of page 4m + g' sit in rows of lane group g'
// (the MFMA writes rows 4g'..4g'+3 to lane group g').  No cross-lane
// reduction is needed per page.
#pragma once

#include "device.h"

namespace kvs {

// Everything one wave loads for its tile: the group's query (B operand; a
// float16 query as an exact bfloat16 hi + lo pair because the summary is
// bfloat16), log n of its pages and every record vector it feeds the MFMA.
template <int D, int R, bool F16>
struct ScoreTile {
  static constexpr int KS = D / 32;
  u32x4_t qh[KS];
  u32x4_t ql[F16 ? KS : 1];
  float ln[4];
  u32x4_t a[1 + R][KS];
};

// Requests the tile of 16 pages [base, base + 16) of row (b, g).  Pages past
// max_pages read a clamped, always allocated record and their results are
// dropped, so every load is unconditional.
template <int D, int R, bool F16>
__device__ __forceinline__ void score_tile_issue(ScoreTile<D, R, F16>& t, const uint16_t* __restrict__ q,
                                                 const uint16_t* __restrict__ summary,
                                                 const float* __restrict__ log_n, int b, int g, int Hkv, int G,
                                                 int max_pages, int base) {
  constexpr int KS = D / 32;
  constexpr int REC = (1 + R) * D;
  constexpr int PPL = (R <= 4) ? 4 / R : 1;   // pages per lane group in one direction tile
  const int lane = threadIdx.x & 63;
  const int col = lane & 15;   // A row within the tile; also the output column (= head)
  const int kg = lane >> 4;    // A k-group; also the output row group
  const int row = b * Hkv + g;
  auto clampp = [&](int p) { return p < max_pages ? p : max_pages - 1; };

#pragma unroll
  for (int m = 0; m < 4; ++m) t.ln[m] = log_n[(size_t)b * max_pages + clampp(base + 4 * m + kg)];

  // Element assignment: at k-step s, k-group kg holds head-dim elements
  // [32s + 8kg, 32s + 8kg + 8), so one load instruction reads 64 contiguous
  // bytes of each of 16 vectors.  The query uses the same assignment.
  {
    const int Hq = Hkv * G;
    const uint16_t* qp = q + ((size_t)b * Hq + (size_t)g * G + (col < G ? col : 0)) * D + 8 * kg;
#pragma unroll
    for (int s = 0; s < KS; ++s) t.qh[s] = ld16(qp + 32 * s);
  }

  // mean tile: A row r = col holds page (r & 3) * 4 + (r >> 2)
  // direction tile wt: A row r holds w_j of page pl (mapping below)
  const uint16_t* rowrec = summary + (size_t)row * max_pages * REC + 8 * kg;
  {
    const uint16_t* src = rowrec + (size_t)clampp(base + (col & 3) * 4 + (col >> 2)) * REC;
#pragma unroll
    for (int s = 0; s < KS; ++s) t.a[0][s] = ld16(src + 32 * s);
  }
#pragma unroll
  for (int wt = 0; wt < R; ++wt) {
    const int gq = col >> 2, i = col & 3;
    int pl, j;
    if constexpr (R <= 4) { pl = 4 * (wt * PPL + i / R) + gq; j = i % R; }
    else { pl = 4 * (wt / 2) + gq; j = 4 * (wt % 2) + i; }
    const uint16_t* src = rowrec + (size_t)clampp(base + pl) * REC + (size_t)(1 + j) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) t.a[1 + wt][s] = ld16(src + 32 * s);
  }
}

// Scores of the tile's pages for every head of the group (written to
// head_scores[row][head][page]; COH: device-coherent stores, for a reader in
// another block of the same launch) and this wave's (max, sum exp) per head,
// merged over the four lane groups: lanes 0..15 hold head `lane`'s pair.
template <int D, int R, bool F16, bool COH>
__device__ __forceinline__ void score_tile_finish(ScoreTile<D, R, F16>& t, int row, int G, int Np,
                                                  int max_pages, int base, float tau,
                                                  float* __restrict__ head_scores, float& run_m, float& run_s) {
  constexpr int KS = D / 32;
  constexpr int PPL = (R <= 4) ? 4 / R : 1;
  const int lane = threadIdx.x & 63;
  const int col = lane & 15, kg = lane >> 4;

  // query heads past G are zero columns
  {
    const uint32_t keep = col < G ? 0xFFFFFFFFu : 0u;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      u32x4_t raw = t.qh[s];
#pragma unroll
      for (int w = 0; w < 4; ++w) raw[w] &= keep;
      if constexpr (!F16) {
        t.qh[s] = raw;
      } else {
        // a float16 query is split exactly into two bfloat16 halves (11 = 8 + 3 bits)
#pragma unroll
        for (int w = 0; w < 4; ++w) {
          const float f0 = f16_bits_to_f32(raw[w] & 0xFFFFu), f1 = f16_bits_to_f32(raw[w] >> 16);
          const uint32_t h0 = __float_as_uint(f0) & 0xFFFF0000u, h1 = __float_as_uint(f1) & 0xFFFF0000u;
          const uint32_t l0 = __float_as_uint(f0 - __uint_as_float(h0)) >> 16;
          const uint32_t l1 = __float_as_uint(f1 - __uint_as_float(h1)) >> 16;
          t.qh[s][w] = (h0 >> 16) | h1;
          t.ql[s][w] = l0 | (l1 << 16);
        }
      }
    }
  }

  f32x4_t acc_mu = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    acc_mu = mfma16<false>(t.a[0][s], t.qh[s], acc_mu);
    if constexpr (F16) acc_mu = mfma16<false>(t.a[0][s], t.ql[s], acc_mu);
  }
  float quad[4] = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int wt = 0; wt < R; ++wt) {
    f32x4_t acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      acc = mfma16<false>(t.a[1 + wt][s], t.qh[s], acc);
      if constexpr (F16) acc = mfma16<false>(t.a[1 + wt][s], t.ql[s], acc);
    }
#pragma unroll
    for (int ii = 0; ii < 4; ++ii) {
      const int m = (R <= 4) ? wt * PPL + ii / R : wt / 2;
      quad[m] += acc[ii] * acc[ii];
    }
  }

  // scores of pages base + 4m + kg for head col
  const float c1 = tau, c2 = 0.5f * tau * tau;
  run_m = -INFINITY;
  run_s = 0.f;
#pragma unroll
  for (int m = 0; m < 4; ++m) {
    const int p = base + 4 * m + kg;
    const float s = p < Np ? t.ln[m] + c1 * acc_mu[m] + c2 * quad[m] : -INFINITY;
    if (col < G && p < max_pages) {
      float* dst = head_scores + ((size_t)row * G + col) * max_pages + p;
      if constexpr (COH) __hip_atomic_store(dst, s, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      else *dst = s;
    }
    if (p < Np && s != -INFINITY) lse_merge(run_m, run_s, s, 1.f);
  }

  // combine the four lane groups (same head) in a fixed order
  float m2 = __shfl_xor(run_m, 16), s2 = __shfl_xor(run_s, 16);
  lse_merge(run_m, run_s, m2, s2);
  m2 = __shfl_xor(run_m, 32);
  s2 = __shfl_xor(run_s, 32);
  lse_merge(run_m, run_s, m2, s2);
}

}  // namespace kvs
