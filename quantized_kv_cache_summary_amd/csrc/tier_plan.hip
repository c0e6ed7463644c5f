// Tier plan along the compression cascade.  ARGUS (argus_cache 0.1.7.1
// project page): "The One-Minute Explanation" (critical, recent and highly
// attended tokens stay in 16-bit; cold memory is compressed step by step from
// FP8 to 1-bit), "Visual Architecture" (the cascade native -> FP8 -> int8 ->
// int4 -> int2 -> 1-bit) and the per-tier page budgets of its configuration.
//
// One block per sequence, over its valid pages p < Np:
//   importance i_p = max over the KV heads of page_S (NaN as -inf); the first
//   n_force_first and last n_force_last pages rank above all others;
//   for each level l < 5 the top cap_0 + ... + cap_l pages (importance
//   descending, page index ascending: the selector's radix search and ordered
//   compaction) count the page as inside that budget; desired level
//   d_p = 5 - (budgets containing p);
//   a page whose desired level is below its current one moves down one
//   level; pages never move up.
// Moves are listed per sequence in page order: (physical page, new tier).

#include "device.h"
#include "launch.h"
#include "select.h"

namespace kvs {

constexpr int kPlanThreads = 512;

__device__ __forceinline__ int level_of_tier(uint32_t t) {
  // native, I8, I4, I2, B1, FP8 -> 0, 2, 3, 4, 5, 1
  return t == KV_TIER_NATIVE ? 0 : t == KV_TIER_FP8 ? 1 : (int)t + 1;
}

__device__ __forceinline__ int tier_of_level(int l) {
  return l == 0 ? KV_TIER_NATIVE : l == 1 ? KV_TIER_FP8 : l - 1;
}

template <int NT>
__global__ __launch_bounds__(NT) void tier_plan_kernel(const float* __restrict__ page_S,
                                                       const int32_t* __restrict__ seq_lens, int Hkv, int P,
                                                       int max_pages, const int32_t* __restrict__ block_table,
                                                       const uint32_t* __restrict__ page_entry, int cap0, int cap1,
                                                       int cap2, int cap3, int cap4, int n_force_first,
                                                       int n_force_last, int32_t* __restrict__ moves,
                                                       int32_t* __restrict__ move_count) {
  constexpr int NW = NT / 64;
  extern __shared__ uint32_t keys[];                       // [max_pages], then inside[] bytes
  uint8_t* inside = reinterpret_cast<uint8_t*>(keys + max_pages);
  __shared__ SelectLds<NT> sh;
  const int b = blockIdx.x, tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int L = seq_lens[b];
  int Np = L > 0 ? (L + P - 1) / P : 0;
  Np = Np < max_pages ? Np : max_pages;

  // keys and their extremes
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  int npos = 0, nneg = 0;
  for (int p = tid; p < Np; p += NT) {
    float imp = -INFINITY;
    for (int g = 0; g < Hkv; ++g) {
      const float v = page_S[((size_t)b * Hkv + g) * max_pages + p];
      imp = v > imp ? v : imp;                              // NaN never wins
    }
    const bool forced = p < n_force_first || p >= Np - n_force_last;
    const uint32_t key = forced ? kKeyPosInf : order_key(imp);
    keys[p] = key;
    inside[p] = 0;
    if (finite_key(key)) {
      kmax = key > kmax ? key : kmax;
      kmin = key < kmin ? key : kmin;
    }
    npos += key == kKeyPosInf;
    nneg += key == kKeyNegInf;
  }
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);
  npos = wave_sum_i32(npos);
  nneg = wave_sum_i32(nneg);
  if (lane == 0) { sh.wmax[wave] = kmax; sh.wmin[wave] = kmin; sh.wpos[wave] = npos; sh.wneg[wave] = nneg; }
  __syncthreads();
  SelectStats st;
  st.kmax = sh.wmax[0];
  st.kmin = sh.wmin[0];
  st.npos = sh.wpos[0];
  st.nneg = sh.wneg[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    st.kmax = sh.wmax[w] > st.kmax ? sh.wmax[w] : st.kmax;
    st.kmin = sh.wmin[w] < st.kmin ? sh.wmin[w] : st.kmin;
    st.npos += sh.wpos[w];
    st.nneg += sh.wneg[w];
  }

  // the five nested budgets
  const int caps[5] = {cap0, cap1, cap2, cap3, cap4};
  int K = 0;
  for (int l = 0; l < 5; ++l) {
    K += caps[l];
    const int k = K < Np ? K : Np;
    __syncthreads();                                        // previous pass done with the shared state
    if (tid == 0) sh.n_cand = 0;
    if (tid < kDirectMax) sh.cand[tid] = 0u;
    if (tid < 256) sh.hist[0][tid] = 0;
    __syncthreads();
    if (k == 0) continue;
    uint32_t T;
    int take;
    select_kth<NT>(sh, keys, Np, st, k, T, take);
    select_compact<NT>(sh, keys, Np, T, take, [&](int p, int) { inside[p] += 1; });
  }
  __syncthreads();

  // moves in page order: each thread owns a contiguous run of pages
  const int chunk = (Np + NT - 1) / NT;
  const int lo = tid * chunk, hi = lo + chunk < Np ? lo + chunk : Np;
  const int32_t* bt = block_table + (size_t)b * max_pages;
  int mine = 0;
  for (int p = lo; p < hi; ++p) {
    const int cur = level_of_tier(page_entry[bt[p]] >> 29);
    mine += (5 - (int)inside[p]) > cur;
  }
  const int incl = wave_incl_sum(mine);
  if (lane == 63) sh.wave_tot[wave] = incl;
  __syncthreads();
  int pos = incl - mine, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) pos += sh.wave_tot[w];
    total += sh.wave_tot[w];
  }
  int32_t* out = moves + (size_t)b * max_pages * 2;
  for (int p = lo; p < hi; ++p) {
    const int phys = bt[p];
    const int cur = level_of_tier(page_entry[phys] >> 29);
    if ((5 - (int)inside[p]) > cur) {
      out[2 * pos] = phys;
      out[2 * pos + 1] = tier_of_level(cur + 1);
      ++pos;
    }
  }
  if (tid == 0) move_count[b] = total;
}

hipError_t launch_tier_plan(const kv_layout& L, const float* page_S, const int32_t* seq_lens, int B,
                            int max_pages, const int32_t* block_table, const uint32_t* page_entry,
                            const int32_t* caps, int n_force_first, int n_force_last, int32_t* moves,
                            int32_t* move_count, hipStream_t st) {
  const size_t lds = (size_t)max_pages * sizeof(uint32_t) + (size_t)max_pages;
  hipError_t e = hipFuncSetAttribute((const void*)tier_plan_kernel<kPlanThreads>,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL((tier_plan_kernel<kPlanThreads>), dim3(B), dim3(kPlanThreads), lds, st, page_S, seq_lens,
                     L.num_kv_heads, L.page_size, max_pages, block_table, page_entry, caps[0], caps[1], caps[2],
                     caps[3], caps[4], n_force_first, n_force_last, moves, move_count);
  return hipGetLastError();
}

}  // namespace kvs
