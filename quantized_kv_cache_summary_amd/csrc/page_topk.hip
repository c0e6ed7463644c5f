// Group aggregation and top-k page selection, one block per (sequence, KV
// head); the selection itself is select_threshold / select_compact.

#include "device.h"
#include "launch.h"
#include "select.h"

namespace kvs {

template <int GM, int NT>
__global__ __launch_bounds__(NT) void page_topk_kernel(
    const float* __restrict__ head_scores, const float* __restrict__ lse_partial,
    const int32_t* __restrict__ seq_lens, int Hkv, int G, int P, int max_pages, int n_tiles,
    float keep, int k_fixed, float coverage, int n_force_first, int n_force_last, int32_t* __restrict__ sel,
    int32_t* __restrict__ sel_count, int k_max, float* __restrict__ page_S) {
  extern __shared__ uint32_t keys[];   // max_pages
  __shared__ SelectLds<NT> sh;

  const int row = blockIdx.x;
  const int b = row / Hkv;
  const int tid = threadIdx.x;
  const float* hs = head_scores + (size_t)row * G * max_pages;
  const float* lsep = lse_partial + (size_t)row * n_tiles * G * 2;
  SelectLoads<NT, GM> ld;
  if (max_pages > 0) select_issue<NT, GM>(ld, hs, lsep, G, max_pages, n_tiles);

  const int L = seq_lens[b];
  int Np = L > 0 ? (L + P - 1) / P : 0;
  Np = Np < max_pages ? Np : max_pages;
  // coverage >= 0: coverage mode, k from the mass prefix (known after the keys)
  const bool cov = coverage >= 0.f;
  int k = cov ? (Np > 0 ? 1 : 0) : selection_count(Np, keep, k_fixed);
  int32_t* out = sel + (size_t)row * k_max;
  if (k == 0) {
    for (int i = tid; i < k_max; i += NT) out[i] = -1;
    if (tid == 0) sel_count[row] = 0;
    return;
  }
  const SelectStats st = select_keys<NT, GM>(sh, keys, ld, hs, G, max_pages, n_tiles, Np, n_force_first,
                                             n_force_last, page_S ? page_S + (size_t)row * max_pages : nullptr,
                                             cov);
  if (cov) {
    k = select_coverage_k<NT>(sh, keys, Np, st, coverage, k_max);
    __syncthreads();                 // every wave is done with the histograms
    if (tid < 256) sh.hist[0][tid] = 0;
    __syncthreads();
  }
  for (int i = k + tid; i < k_max; i += NT) out[i] = -1;
  if (tid == 0) sel_count[row] = k;

  uint32_t T;
  int take;
  select_kth<NT>(sh, keys, Np, st, k, T, take);
  select_compact<NT>(sh, keys, Np, T, take, [&](int p, int pos) {
    if (pos < k) out[pos] = p;
  });
}

hipError_t launch_page_topk(const kv_layout& L, const float* head_scores, const float* lse_partial,
                            const int32_t* seq_lens, int B, int max_pages, float keep, int k_fixed,
                            float coverage, int n_force_first, int n_force_last, int32_t* sel,
                            int32_t* sel_count, int k_max, float* page_S, hipStream_t st) {
  const int G = L.num_q_heads / L.num_kv_heads;
  const int rows = B * L.num_kv_heads;
  const size_t lds = (size_t)(max_pages > 0 ? max_pages : 1) * sizeof(uint32_t);
  // long rows: twice the threads, so twice the head scores are in flight at once
#define KVS_TOPK(GM_, NT_) hipLaunchKernelGGL((page_topk_kernel<GM_, NT_>), dim3(rows), dim3(NT_), lds, st,  \
                     head_scores, lse_partial, seq_lens, L.num_kv_heads, G, L.page_size, max_pages,     \
                     score_tiles(max_pages), keep, k_fixed, coverage, n_force_first, n_force_last, sel, \
                     sel_count, k_max, page_S)
  const bool wide = max_pages >= kTopkWideFrom;
  if (G <= 4) { if (wide) KVS_TOPK(4, 2 * kTopkThreads); else KVS_TOPK(4, kTopkThreads); }
  else if (G <= 8) { if (wide) KVS_TOPK(8, 2 * kTopkThreads); else KVS_TOPK(8, kTopkThreads); }
  else { if (wide) KVS_TOPK(16, 2 * kTopkThreads); else KVS_TOPK(16, kTopkThreads); }
#undef KVS_TOPK
  return hipGetLastError();
}

}  // namespace kvs
