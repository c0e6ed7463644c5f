// Quad page score from shared-basis summaries.  AMASS (amass-kv 0.1.1 project
// page), "What is in the box" item 1 (a quadratic Gaussian-MGF score from a
// per-page summary that keeps only r' eigen-quantities) and "Benchmarking"
// (the score stage is bandwidth-bound).  For every logical page p of a
// (sequence, KV head) row and every query head h of its group:
//   s = log n_p + tau q_h.mu_p + (tau^2 / 2) sum_j lam_pj (q_h.u_j)^2
// with u the row's float32 basis, mu bfloat16, lam and log n float32.
//
// gfx950 design.  The stream is the page means (d bfloat16 per page): a wave
// owns 64 pages (four 16-page MFMA tiles, q.mu as in the per-page score
// kernel: mean vectors are the A rows, the group's heads the B columns) and
// issues all of their loads before any math.  The page variances and log n
// of the wave's 64 pages arrive as one load per lane and are shared through
// LDS, so only the means hold registers while in flight.  c_hj = q_h.u_j is
// computed once per wave with the same MFMA shape: the float32 basis rows are
// split exactly into three bfloat16 parts (8 + 8 + 8 significand bits), so
// the products are exact and only the float32 accumulation rounds.  Each wave
// emits the (max, sum exp) of its 64 pages per head, the partial the selector
// merges.

#include "device.h"
#include "launch.h"

namespace kvs {

constexpr int kBasisScoreWaves = 4;   // 64-page chunks per block

// Exact split of float32 values into three bfloat16 parts (truncation).
__device__ __forceinline__ void split3_bf16(float x0, float x1, uint32_t& h, uint32_t& m, uint32_t& l) {
  const uint32_t u0 = __float_as_uint(x0) & 0xFFFF0000u, u1 = __float_as_uint(x1) & 0xFFFF0000u;
  const float r0 = x0 - __uint_as_float(u0), r1 = x1 - __uint_as_float(u1);
  const uint32_t v0 = __float_as_uint(r0) & 0xFFFF0000u, v1 = __float_as_uint(r1) & 0xFFFF0000u;
  const float t0 = r0 - __uint_as_float(v0), t1 = r1 - __uint_as_float(v1);
  h = (u0 >> 16) | u1;
  m = (v0 >> 16) | v1;
  l = (__float_as_uint(t0) >> 16) | (__float_as_uint(t1) & 0xFFFF0000u);
}

template <int D, int R, bool F16>
__global__ __launch_bounds__(64 * kBasisScoreWaves) void page_score_basis_kernel(
    const uint16_t* __restrict__ q, const uint16_t* __restrict__ mu, const float* __restrict__ lam,
    const float* __restrict__ basis, const float* __restrict__ log_n, const int32_t* __restrict__ seq_lens,
    int Hkv, int G, int P, int max_pages, int n_tiles, float tau, float* __restrict__ head_scores,
    float* __restrict__ lse_partial) {
  constexpr int KS = D / 32;   // MFMA k-steps per vector
  constexpr int SUB = kScorePagesPerBlock / 16;   // 16-page tiles per wave
  __shared__ float lamL[kBasisScoreWaves][kScorePagesPerBlock][R];
  __shared__ float lnL[kBasisScoreWaves][kScorePagesPerBlock];

  const int row = blockIdx.y;
  const int b = row / Hkv, g = row - b * Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int col = lane & 15;   // A row within a tile; also the output column (= head)
  const int kg = lane >> 4;    // A k-group; also the output row group
  const int chunk = blockIdx.x * kBasisScoreWaves + wave;
  if (chunk >= n_tiles) return;   // whole wave; this kernel has no block barrier
  const int base = chunk * kScorePagesPerBlock;
  auto clampp = [&](int p) { return p < max_pages ? p : max_pages - 1; };

  // ---- every load of the wave, before any math: first the small ones the
  //      basis projections need, so that work overlaps the means in flight
  const size_t rrow = (size_t)row * max_pages;
  // query operand: head `col`, elements [32s + 8kg, +8); heads past G are zero
  u32x4_t qraw[KS];
  {
    const uint16_t* qp = q + ((size_t)b * Hkv * G + (size_t)g * G + (col < G ? col : 0)) * D + 8 * kg;
#pragma unroll
    for (int s = 0; s < KS; ++s) qraw[s] = ld16(qp + 32 * s);
  }
  // basis operand: row j = col (< R), the same element assignment
  float ub[KS][8];
  {
    const float* up = basis + ((size_t)row * R + (col < R ? col : R - 1)) * D + 8 * kg;
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      const float4 x0 = *reinterpret_cast<const float4*>(up + 32 * s);
      const float4 x1 = *reinterpret_cast<const float4*>(up + 32 * s + 4);
      ub[s][0] = x0.x; ub[s][1] = x0.y; ub[s][2] = x0.z; ub[s][3] = x0.w;
      ub[s][4] = x1.x; ub[s][5] = x1.y; ub[s][6] = x1.z; ub[s][7] = x1.w;
    }
  }
  float lv[R];
  {
    const float* lp = lam + (rrow + clampp(base + lane)) * R;
#pragma unroll
    for (int j = 0; j < R; ++j) lv[j] = lp[j];
  }
  const float lnv = log_n[(size_t)b * max_pages + clampp(base + lane)];
  const int L = seq_lens[b];
  const uint16_t* mrow = mu + rrow * D + 8 * kg;
  u32x4_t a[SUB][KS];
#pragma unroll
  for (int t = 0; t < SUB; ++t) {
    const uint16_t* src = mrow + (size_t)clampp(base + 16 * t + (col & 3) * 4 + (col >> 2)) * D;
#pragma unroll
    for (int s = 0; s < KS; ++s) a[t][s] = ld16(src + 32 * s);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- page variances and log n of the wave's 64 pages through LDS
#pragma unroll
  for (int j = 0; j < R; ++j) lamL[wave][lane][j] = lv[j];
  lnL[wave][lane] = lnv;

  // ---- query operands
  u32x4_t qh[KS], ql[KS];
  const uint32_t keep = col < G ? 0xFFFFFFFFu : 0u;
#pragma unroll
  for (int s = 0; s < KS; ++s) {
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      const uint32_t raw = qraw[s][w] & keep;
      if constexpr (!F16) {
        qh[s][w] = raw;
      } else {
        // a float16 query is split exactly into two bfloat16 halves
        const float f0 = f16_bits_to_f32(raw & 0xFFFFu), f1 = f16_bits_to_f32(raw >> 16);
        const uint32_t h0 = __float_as_uint(f0) & 0xFFFF0000u, h1 = __float_as_uint(f1) & 0xFFFF0000u;
        const uint32_t l0 = __float_as_uint(f0 - __uint_as_float(h0)) >> 16;
        const uint32_t l1 = __float_as_uint(f1 - __uint_as_float(h1)) >> 16;
        qh[s][w] = (h0 >> 16) | h1;
        ql[s][w] = l0 | (l1 << 16);
      }
    }
  }

  // ---- c[h][j] = q_h . u_j: lane (h, kg) receives rows j = 4kg + i
  f32x4_t cacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    u32x4_t uh, um, ul;
#pragma unroll
    for (int w = 0; w < 4; ++w) {
      float x0 = ub[s][2 * w], x1 = ub[s][2 * w + 1];
      if (col >= R) { x0 = 0.f; x1 = 0.f; }
      uint32_t hh, mm, ll;
      split3_bf16(x0, x1, hh, mm, ll);
      uh[w] = hh; um[w] = mm; ul[w] = ll;
    }
    cacc = mfma16<false>(uh, qh[s], cacc);
    cacc = mfma16<false>(um, qh[s], cacc);
    cacc = mfma16<false>(ul, qh[s], cacc);
    if constexpr (F16) {
      cacc = mfma16<false>(uh, ql[s], cacc);
      cacc = mfma16<false>(um, ql[s], cacc);
      cacc = mfma16<false>(ul, ql[s], cacc);
    }
  }
  const float c2 = 0.5f * tau * tau;
  float csq[R];
#pragma unroll
  for (int j = 0; j < R; ++j) {
    const float cj = __shfl(cacc[j & 3], col + 16 * (j >> 2));
    csq[j] = c2 * cj * cj;
  }

  // ---- q . mu for the four tiles
  f32x4_t acc[SUB];
#pragma unroll
  for (int t = 0; t < SUB; ++t) {
    acc[t] = f32x4_t{0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < KS; ++s) {
      acc[t] = mfma16<false>(a[t][s], qh[s], acc[t]);
      if constexpr (F16) acc[t] = mfma16<false>(a[t][s], ql[s], acc[t]);
    }
  }
  wave_lds_sync();

  // ---- scores of pages base + 16t + 4m + kg for head col
  int Np = L > 0 ? (L + P - 1) / P : 0;
  Np = Np < max_pages ? Np : max_pages;
  float run_m = -INFINITY, run_s = 0.f;
#pragma unroll
  for (int t = 0; t < SUB; ++t) {
#pragma unroll
    for (int m = 0; m < 4; ++m) {
      const int pl = 16 * t + 4 * m + kg;
      const int p = base + pl;
      float quad = 0.f;
#pragma unroll
      for (int j = 0; j < R; ++j) quad = __builtin_fmaf(lamL[wave][pl][j], csq[j], quad);
      const float sc = p < Np ? lnL[wave][pl] + tau * acc[t][m] + quad : -INFINITY;
      if (col < G && p < max_pages) head_scores[((size_t)row * G + col) * max_pages + p] = sc;
      if (p < Np && sc != -INFINITY) lse_merge(run_m, run_s, sc, 1.f);
    }
  }
  // combine the four lane groups (same head) in a fixed order
  {
    float m2 = __shfl_xor(run_m, 16), s2 = __shfl_xor(run_s, 16);
    lse_merge(run_m, run_s, m2, s2);
    m2 = __shfl_xor(run_m, 32);
    s2 = __shfl_xor(run_s, 32);
    lse_merge(run_m, run_s, m2, s2);
  }
  if (lane < G) {
    float* dst = lse_partial + (((size_t)row * n_tiles + chunk) * G + lane) * 2;
    dst[0] = run_m;
    dst[1] = run_s;
  }
}

template <int D, int R, bool F16>
static hipError_t launch_score_basis_t(const kv_layout& L, const void* q, const void* mu, const float* lam,
                                       const float* basis, const float* log_n, const int32_t* sl, int B,
                                       int max_pages, float tau, float* hs, float* lp, hipStream_t st) {
  const int G = L.num_q_heads / L.num_kv_heads;
  const int n_tiles = score_tiles(max_pages);
  const dim3 grid((n_tiles + kBasisScoreWaves - 1) / kBasisScoreWaves, B * L.num_kv_heads);
  hipLaunchKernelGGL((page_score_basis_kernel<D, R, F16>), grid, dim3(64 * kBasisScoreWaves), 0, st,
                     (const uint16_t*)q, (const uint16_t*)mu, lam, basis, log_n, sl, L.num_kv_heads, G,
                     L.page_size, max_pages, n_tiles, tau, hs, lp);
  return hipGetLastError();
}

template <int D, bool F16>
static hipError_t launch_score_basis_r(const kv_layout& L, const void* q, const void* mu, const float* lam,
                                       const float* basis, const float* log_n, const int32_t* sl, int B,
                                       int max_pages, float tau, float* hs, float* lp, hipStream_t st) {
  switch (L.rank) {
    case 1: return launch_score_basis_t<D, 1, F16>(L, q, mu, lam, basis, log_n, sl, B, max_pages, tau, hs, lp, st);
    case 2: return launch_score_basis_t<D, 2, F16>(L, q, mu, lam, basis, log_n, sl, B, max_pages, tau, hs, lp, st);
    case 4: return launch_score_basis_t<D, 4, F16>(L, q, mu, lam, basis, log_n, sl, B, max_pages, tau, hs, lp, st);
    default: return launch_score_basis_t<D, 8, F16>(L, q, mu, lam, basis, log_n, sl, B, max_pages, tau, hs, lp, st);
  }
}

hipError_t launch_page_score_basis(const kv_layout& L, const void* q, const void* mu, const float* lam,
                                   const float* basis, const float* log_n, const int32_t* seq_lens, int B,
                                   int max_pages, float tau, float* head_scores, float* lse_partial,
                                   hipStream_t st) {
  const bool f16 = L.kv_dtype == KV_F16;
  if (L.head_dim == 64)
    return f16 ? launch_score_basis_r<64, true>(L, q, mu, lam, basis, log_n, seq_lens, B, max_pages, tau, head_scores, lse_partial, st)
               : launch_score_basis_r<64, false>(L, q, mu, lam, basis, log_n, seq_lens, B, max_pages, tau, head_scores, lse_partial, st);
  return f16 ? launch_score_basis_r<128, true>(L, q, mu, lam, basis, log_n, seq_lens, B, max_pages, tau, head_scores, lse_partial, st)
             : launch_score_basis_r<128, false>(L, q, mu, lam, basis, log_n, seq_lens, B, max_pages, tau, head_scores, lse_partial, st);
}

}  // namespace kvs
