// Group aggregation and top-k page selection, one block per (sequence, KV head).
// AMASS (amass-kv 0.1.1 project page), "Quickstart" (budget: a fixed selected
// page fraction) and "Benchmarking" (the top-B stage).
//
//   L_h = logsumexp_p s[h][p]                 (merged from the score blocks'
//                                              (max, sum exp) partials)
//   S_p = log((1/G) sum_h exp(s[h][p] - L_h))  (group-mean mass fraction)
//
// Selection is an exact k-th-largest search on order-preserving uint32 keys:
// four 8-bit radix passes with LDS histograms (integer counts, so the result
// does not depend on thread timing), then one ordered compaction that keeps
// every key above the threshold and the lowest-index pages among keys equal
// to it.  Pages come out in ascending order with no sort.  Ties therefore
// break by (S descending, page ascending) exactly.

#include "device.h"
#include "launch.h"

namespace kvs {

constexpr int kTopkWaves = kTopkThreads / 64;
// Key of -inf; NaN scores take it too, so they rank with -inf.
constexpr uint32_t kKeyNegInf = 0x007FFFFFu;

__device__ __forceinline__ uint32_t order_key(float S) {
  if (S != S) return kKeyNegInf;
  S = S + 0.0f;   // -0 -> +0
  const uint32_t u = __float_as_uint(S);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// Exclusive prefix sum over the block (kTopkThreads threads); also returns the total.
__device__ __forceinline__ int block_exclusive_scan(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  int x = v;
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const int y = __shfl_up(x, off);
    if (lane >= off) x += y;
  }
  if (lane == 63) wave_tot[wave] = x;
  __syncthreads();
  int before = 0;
  total = 0;
#pragma unroll
  for (int w = 0; w < kTopkWaves; ++w) {
    const int t = wave_tot[w];
    if (w < wave) before += t;
    total += t;
  }
  __syncthreads();
  return before + x - v;
}

__global__ __launch_bounds__(kTopkThreads) void page_topk_kernel(
    const float* __restrict__ head_scores, const float* __restrict__ lse_partial,
    const int32_t* __restrict__ seq_lens, int Hkv, int G, int P, int max_pages, int n_tiles,
    float keep, int k_fixed, int n_force_first, int n_force_last, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count, int k_max, float* __restrict__ page_S) {
  extern __shared__ uint32_t keys[];   // max_pages
  __shared__ float Lh[16];
  __shared__ int hist[256];
  __shared__ int wave_tot[kTopkWaves];
  __shared__ int digit_sel, digit_above;

  const int row = blockIdx.x;
  const int b = row / Hkv;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int L = seq_lens[b];
  int Np = L > 0 ? (L + P - 1) / P : 0;
  Np = Np < max_pages ? Np : max_pages;

  int k;
  if (Np <= 0) k = 0;
  else if (k_fixed > 0) k = k_fixed < Np ? k_fixed : Np;
  else {
    k = (int)ceil((double)keep * (double)Np);
    k = k < 1 ? 1 : (k > Np ? Np : k);
  }
  int32_t* out = sel + (size_t)row * k_max;
  for (int i = k + tid; i < k_max; i += kTopkThreads) out[i] = -1;
  if (tid == 0) sel_count[row] = k;
  if (k == 0) return;

  // 1. per-head normaliser from the score blocks' partials (fixed merge order)
  for (int h = wave; h < G; h += kTopkWaves) {
    float m = -INFINITY, s = 0.f;
    for (int t = lane; t < n_tiles; t += 64) {
      const float* pp = lse_partial + (((size_t)row * n_tiles + t) * G + h) * 2;
      lse_merge(m, s, pp[0], pp[1]);
    }
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const float m2 = __shfl_xor(m, off), s2 = __shfl_xor(s, off);
      lse_merge(m, s, m2, s2);
    }
    if (lane == 0) Lh[h] = (s > 0.f) ? m + __logf(s) : -INFINITY;
  }
  __syncthreads();

  // 2. group aggregate and keys
  const float logG = __logf((float)G);
  const float* hs = head_scores + (size_t)row * G * max_pages;
  for (int p = tid; p < Np; p += kTopkThreads) {
    float a[16];
    float M = -INFINITY;
    for (int h = 0; h < G; ++h) {
      a[h] = hs[(size_t)h * max_pages + p] - Lh[h];
      M = fmaxf(M, a[h]);
    }
    float S;
    if (M == -INFINITY) {
      S = -INFINITY;
      for (int h = 0; h < G; ++h) if (a[h] != a[h]) S = a[h];
    } else {
      float sum = 0.f;
      for (int h = 0; h < G; ++h) sum += __expf(a[h] - M);
      S = M + __logf(sum) - logG;
    }
    if (p < n_force_first || p >= Np - n_force_last) S = INFINITY;
    keys[p] = order_key(S);
    if (page_S) page_S[(size_t)row * max_pages + p] = S;
  }
  __syncthreads();

  // 3. k-th largest key by four 8-bit radix passes
  uint32_t prefix = 0, pmask = 0;
  int rem = k;
  for (int shift = 24; shift >= 0; shift -= 8) {
    if (tid < 256) hist[tid] = 0;
    __syncthreads();
    for (int p = tid; p < Np; p += kTopkThreads) {
      const uint32_t key = keys[p];
      if ((key & pmask) == prefix) atomicAdd(&hist[(key >> shift) & 255u], 1);
    }
    __syncthreads();
    if (wave == 0) {
      // lane l owns digits 255-4l .. 252-4l (descending)
      int c[4], tot = 0;
#pragma unroll
      for (int i = 0; i < 4; ++i) { c[i] = hist[255 - 4 * lane - i]; tot += c[i]; }
      int incl = tot;
#pragma unroll
      for (int off = 1; off < 64; off <<= 1) {
        const int y = __shfl_up(incl, off);
        if (lane >= off) incl += y;
      }
      const unsigned long long hit = __ballot(incl >= rem);
      const int first = __ffsll((long long)hit) - 1;
      if (lane == first) {
        int cum = incl - tot;
        int dsel = 255 - 4 * lane - 3;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          if (cum + c[i] >= rem) { dsel = 255 - 4 * lane - i; break; }
          cum += c[i];
        }
        digit_sel = dsel;
        digit_above = cum;
      }
    }
    __syncthreads();
    prefix |= (uint32_t)digit_sel << shift;
    pmask |= 0xFFu << shift;
    rem -= digit_above;
    __syncthreads();
  }
  const uint32_t T = prefix;   // k-th largest key; take `rem` of the keys equal to it

  // 4. ordered compaction, pages ascending
  const int chunk = (Np + kTopkThreads - 1) / kTopkThreads;
  const int lo = tid * chunk;
  const int hi = lo + chunk < Np ? lo + chunk : Np;
  int n_gt = 0, n_eq = 0;
  for (int p = lo; p < hi; ++p) {
    const uint32_t key = keys[p];
    n_gt += key > T;
    n_eq += key == T;
  }
  int tot;
  const int eq_before = block_exclusive_scan(n_eq, wave_tot, tot);
  int take_eq = rem - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > n_eq ? n_eq : take_eq);
  const int pos0 = block_exclusive_scan(n_gt + take_eq, wave_tot, tot);
  int pos = pos0, taken = 0;
  for (int p = lo; p < hi; ++p) {
    const uint32_t key = keys[p];
    if (key > T || (key == T && taken < take_eq)) {
      out[pos++] = p;
      taken += key == T;
    }
  }
}

hipError_t launch_page_topk(const kv_layout& L, const float* head_scores, const float* lse_partial,
                            const int32_t* seq_lens, int B, int max_pages, float keep, int k_fixed,
                            int n_force_first, int n_force_last, int32_t* sel, int32_t* sel_count,
                            int k_max, float* page_S, hipStream_t st) {
  const int G = L.num_q_heads / L.num_kv_heads;
  const int rows = B * L.num_kv_heads;
  const size_t lds = (size_t)(max_pages > 0 ? max_pages : 1) * sizeof(uint32_t);
  hipLaunchKernelGGL(page_topk_kernel, dim3(rows), dim3(kTopkThreads), lds, st, head_scores,
                     lse_partial, seq_lens, L.num_kv_heads, G, L.page_size, max_pages,
                     score_tiles(max_pages), keep, k_fixed, n_force_first, n_force_last, sel,
                     sel_count, k_max, page_S);
  return hipGetLastError();
}

}  // namespace kvs
