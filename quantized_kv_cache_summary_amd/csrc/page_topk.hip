// Group aggregation and top-k page selection, one block per (sequence, KV head).
// AMASS (amass-kv 0.1.1 project page), "Quickstart" (budget: a fixed selected
// page fraction) and "Benchmarking" (the top-B stage).
//
//   L_h = logsumexp_p s[h][p]                 (merged from the score blocks'
//                                              (max, sum exp) partials)
//   S_p = log((1/G) sum_h exp(s[h][p] - L_h))  (group-mean mass fraction)
//
// Selection is an exact k-th-largest search on order-preserving uint32 keys:
// 8-bit radix passes with LDS histograms (integer counts, so the result does
// not depend on thread timing) that start at the highest bit in which the
// row's largest and smallest keys differ -- the scores of a row share sign and
// exponent bits, and a first digit taken there would pile every key onto one
// or two histogram bins -- then one ordered compaction that keeps
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
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
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

template <int GM>
__global__ __launch_bounds__(kTopkThreads) void page_topk_kernel(
    const float* __restrict__ head_scores, const float* __restrict__ lse_partial,
    const int32_t* __restrict__ seq_lens, int Hkv, int G, int P, int max_pages, int n_tiles,
    float keep, int k_fixed, int n_force_first, int n_force_last, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count, int k_max, float* __restrict__ page_S) {
  extern __shared__ uint32_t keys[];   // max_pages
  __shared__ float Lh[16];
  __shared__ int hist[2][256];
  __shared__ int wave_tot[kTopkWaves];
  __shared__ uint32_t wave_max[kTopkWaves], wave_min[kTopkWaves];
  __shared__ int digit_sel, digit_above;

  const int row = blockIdx.x;
  const int b = row / Hkv;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // wave-uniform (SGPR)
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

  // 1. the first round of head scores is requested before the per-head
  //    normalisers are merged, so the two loads overlap
  const float* hs = head_scores + (size_t)row * G * max_pages;
  constexpr int U = 4;
  float v[U][GM];
  auto load_round = [&](int p0) {
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * kTopkThreads;
#pragma unroll
      for (int h = 0; h < GM; ++h)   // clamped, always in bounds; extra values are ignored
        v[u][h] = hs[(size_t)(h < G ? h : 0) * max_pages + (p < Np ? p : Np - 1)];
    }
  };
  load_round(tid);
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

  // 2. group aggregate and keys, U pages per thread per round
  const float logG = __logf((float)G);
  float Lr[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) Lr[h] = h < G ? Lh[h] : 0.f;
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  for (int p0 = tid; p0 < Np; p0 += kTopkThreads * U) {
    if (p0 != tid) load_round(p0);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = p0 + u * kTopkThreads;
      if (p >= Np) break;
      float M = -INFINITY;
      bool nan = false;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        if (h < G) {
          v[u][h] -= Lr[h];
          nan |= v[u][h] != v[u][h];
          M = fmaxf(M, v[u][h]);
        }
      }
      float S;
      if (nan) S = __int_as_float(0x7FC00000);
      else if (M == -INFINITY) S = -INFINITY;
      else {
        float sum = 0.f;
#pragma unroll
        for (int h = 0; h < GM; ++h) if (h < G) sum += __expf(v[u][h] - M);
        S = M + __logf(sum) - logG;
      }
      if (p < n_force_first || p >= Np - n_force_last) S = INFINITY;
      const uint32_t key = order_key(S);
      keys[p] = key;
      kmax = key > kmax ? key : kmax;
      kmin = key < kmin ? key : kmin;
      if (page_S) page_S[(size_t)row * max_pages + p] = S;
    }
  }
  // block max / min of the keys: the radix passes start below their common prefix
#pragma unroll
  for (int off = 1; off < 64; off <<= 1) {
    const uint32_t a = (uint32_t)__shfl_xor((int)kmax, off), c = (uint32_t)__shfl_xor((int)kmin, off);
    kmax = a > kmax ? a : kmax;
    kmin = c < kmin ? c : kmin;
  }
  if (lane == 0) { wave_max[wave] = kmax; wave_min[wave] = kmin; }
  __syncthreads();
  kmax = wave_max[0];
  kmin = wave_min[0];
#pragma unroll
  for (int w = 1; w < kTopkWaves; ++w) {
    kmax = wave_max[w] > kmax ? wave_max[w] : kmax;
    kmin = wave_min[w] < kmin ? wave_min[w] : kmin;
  }

  // 3. k-th largest key: 8-bit radix passes from the highest differing bit down
  uint32_t prefix = kmax & ~0u, pmask = 0;
  int rem = k;
  const uint32_t diff = kmax ^ kmin;
  if (diff == 0) {
    prefix = kmax;               // every key equal
  } else {
    const int hb = 31 - __clz((int)diff);
    pmask = hb >= 31 ? 0u : ~((2u << hb) - 1u);   // common prefix bits
    prefix = kmax & pmask;
    int top = hb;                                   // highest bit of the next digit
    int buf = 0;
    if (tid < 256) hist[0][tid] = 0;
    __syncthreads();
    while (top >= 0) {
      const int width = top + 1 < 8 ? top + 1 : 8;
      const int shift = top + 1 - width;
      const uint32_t dmask = (1u << width) - 1u;
      for (int p = tid; p < Np; p += kTopkThreads) {
        const uint32_t key = keys[p];
        if ((key & pmask) == prefix) atomicAdd(&hist[buf][(key >> shift) & dmask], 1);
      }
      if (tid < 256) hist[buf ^ 1][tid] = 0;     // clear the other buffer for the next pass
      __syncthreads();
      if (wave == 0) {
        // lane l owns digits 255-4l .. 252-4l (descending); unused digits are 0
        int c[4], tot = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) { c[i] = hist[buf][255 - 4 * lane - i]; tot += c[i]; }
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
      pmask |= dmask << shift;
      rem -= digit_above;
      buf ^= 1;
      top -= width;
    }
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
#define KVS_TOPK(GM_) hipLaunchKernelGGL((page_topk_kernel<GM_>), dim3(rows), dim3(kTopkThreads), lds, st, \
                     head_scores, lse_partial, seq_lens, L.num_kv_heads, G, L.page_size, max_pages,     \
                     score_tiles(max_pages), keep, k_fixed, n_force_first, n_force_last, sel,           \
                     sel_count, k_max, page_S)
  if (G <= 4) KVS_TOPK(4);
  else if (G <= 8) KVS_TOPK(8);
  else KVS_TOPK(16);
#undef KVS_TOPK
  return hipGetLastError();
}

}  // namespace kvs
