// Hot-buffer admission for a host-resident value pool.  AMASS (amass-kv 0.1.1
// project page), "What is in the box" item 2 and the AMASS-mem variant: V in
// pinned, device-mapped host memory with a bounded resident hot buffer and a
// staging pool; only the pages a step calls stay in device memory.
//
// Once per step, after its attention, with U = the physical pages the step's
// selections name (entries i < sel_count of pages p < Np_b, through the block
// table), with no duplicates:
//   1. a page of U already hot has its slot stamped with the step;
//   2. the pages of U not hot, ascending by page id, go to the slots least
//      recently used before this step (smallest (stamp, slot index) among
//      slots stamped below the step), one per slot, paired in ascending slot
//      order; with fewer such slots than pages, the lowest page ids win;
//   3. an admitted slot drops its old page, takes the new one, is stamped, and
//      the page's V (every KV head) is copied in from the pool; with a K hot
//      buffer (the mem-kv variant: K offloaded as well) its K too.
//
// One block plans the step: U as a bitmap in LDS (integer atomics), the misses
// by an ordered compaction of the bitmap, the victim slots as the k largest of
// the keys 0xFF7FFFFF - stamp with the selector's radix search and ordered
// compaction (ties by slot index).  A second kernel copies the admitted pages.

#include "device.h"
#include "launch.h"
#include "select.h"

namespace kvs {

constexpr int kAdmitThreads = 1024;

// Workspace: [0] number of copies, then (page, slot) pairs.
__global__ __launch_bounds__(kAdmitThreads) void hot_admit_plan_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int B, int Hkv, int P,
    int max_pages, const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int k_max,
    int32_t* __restrict__ hot, int n_phys, int32_t* __restrict__ slot_page, uint32_t* __restrict__ slot_stamp,
    int n_slots, uint32_t step, int32_t* __restrict__ ws) {
  constexpr int NT = kAdmitThreads;
  constexpr int NW = NT / 64;
  extern __shared__ uint32_t dyn[];
  const int n_words = (n_phys + 31) >> 5;
  uint32_t* bits = dyn;                 // [n_words] pages of U
  uint32_t* keys = dyn + n_words;       // [n_slots] victim keys
  __shared__ SelectLds<NT> sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  for (int w = tid; w < n_words; w += NT) bits[w] = 0u;
  if (tid == 0) sh.n_cand = 0;
  if (tid < kDirectMax) sh.cand[tid] = 0u;
  if (tid < 256) sh.hist[0][tid] = 0;
  __syncthreads();

  // 1. U: every valid selection entry, through the block table; a thread
  //    takes kBatch entries at a time so their loads are in flight together
  constexpr int kBatch = 16;
  const size_t n_entries = (size_t)B * Hkv * k_max;
  for (size_t e0 = tid; e0 < n_entries; e0 += (size_t)NT * kBatch) {
    int p[kBatch], b[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const size_t e = e0 + (size_t)j * NT;
      p[j] = -1;
      b[j] = 0;
      if (e < n_entries) {
        const int row = (int)(e / k_max), i = (int)(e - (size_t)row * k_max);
        int cnt = sel_count[row];
        cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
        b[j] = row / Hkv;
        if (i < cnt) p[j] = sel[e];
      }
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const int L = seq_lens[b[j]];
      int Np = L > 0 ? (L + P - 1) / P : 0;
      Np = Np < max_pages ? Np : max_pages;
      p[j] = p[j] >= 0 && p[j] < Np ? block_table[(size_t)b[j] * max_pages + p[j]] : -1;
    }
#pragma unroll
    for (int j = 0; j < kBatch; ++j)
      if (p[j] >= 0 && p[j] < n_phys) atomicOr(&bits[p[j] >> 5], 1u << (p[j] & 31));
  }
  __syncthreads();

  // 2. hits get the step's stamp; each word of the bitmap is replaced by its
  //    misses (the hot-map loads of a word are in flight together), then the
  //    misses are listed ascending (each thread owns a contiguous run of words)
  const int chunk = (n_words + NT - 1) / NT;
  const int w0 = tid * chunk, w1 = w0 + chunk < n_words ? w0 + chunk : n_words;
  int my_miss = 0;
  for (int w = w0; w < w1; ++w) {
    const uint32_t m = bits[w];
    if (m == 0u) continue;
    int hs[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) hs[j] = (m >> j) & 1u ? hot[(w << 5) + j] : 0;
    uint32_t miss = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      if (!((m >> j) & 1u)) continue;
      const int sl = hs[j];
      if (sl >= 0 && sl < n_slots) slot_stamp[sl] = step;
      else miss |= 1u << j;
    }
    bits[w] = miss;
    my_miss += __popc(miss);
  }
  // exclusive scan of the miss counts over the block
  const int incl = wave_incl_sum(my_miss);
  if (lane == 63) sh.wave_tot[wave] = incl;
  __syncthreads();
  int before = incl - my_miss, total = 0;
#pragma unroll
  for (int w = 0; w < NW; ++w) {
    if (w < wave) before += sh.wave_tot[w];
    total += sh.wave_tot[w];
  }
  int32_t* miss = ws + 1 + 2 * n_slots;   // the first n_slots misses, ascending
  int pos = before;
  for (int w = w0; w < w1 && pos < n_slots; ++w) {
    uint32_t m = bits[w];
    while (m && pos < n_slots) {
      const int bit = __ffs((int)m) - 1;
      m &= m - 1u;
      miss[pos++] = (w << 5) + bit;
    }
  }
  __syncthreads();   // hit stamps and the miss list are visible to the block

  // 3. victim slots: keys 0xFF7FFFFF - stamp for slots stamped below the step
  //    (larger key = older), the others at the -inf key
  int n_free = 0;
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  for (int s = tid; s < n_slots; s += NT) {
    const uint32_t st = slot_stamp[s];
    uint32_t key = kKeyNegInf;
    if (st < step) {
      key = 0xFF7FFFFFu - (st < 0xFEFFFFFFu ? st : 0xFEFFFFFFu);
      ++n_free;
      kmax = key > kmax ? key : kmax;
      kmin = key < kmin ? key : kmin;
    }
    keys[s] = key;
  }
  n_free = wave_sum_i32(n_free);
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);
  if (lane == 0) { sh.wpos[wave] = n_free; sh.wmax[wave] = kmax; sh.wmin[wave] = kmin; }
  __syncthreads();
  SelectStats st;
  st.kmax = sh.wmax[0];
  st.kmin = sh.wmin[0];
  st.npos = 0;
  n_free = sh.wpos[0];
#pragma unroll
  for (int w = 1; w < NW; ++w) {
    st.kmax = sh.wmax[w] > st.kmax ? sh.wmax[w] : st.kmax;
    st.kmin = sh.wmin[w] < st.kmin ? sh.wmin[w] : st.kmin;
    n_free += sh.wpos[w];
  }
  st.nneg = n_slots - n_free;
  int n = total < n_free ? total : n_free;
  n = n < n_slots ? n : n_slots;
  if (tid == 0) ws[0] = n;
  if (n == 0) return;
  uint32_t T;
  int take;
  select_kth<NT>(sh, keys, n_slots, st, n, T, take);

  // 4. pair the i-th victim (ascending slot) with the i-th miss (ascending page)
  select_compact<NT>(sh, keys, n_slots, T, take, [&](int s, int i) {
    if (i >= n) return;
    const int p = miss[i];
    const int old = slot_page[s];
    if (old >= 0 && old < n_phys) hot[old] = -1;
    slot_page[s] = p;
    hot[p] = s;
    slot_stamp[s] = step;
    ws[1 + 2 * i] = p;
    ws[2 + 2 * i] = s;
  });
}

// Copies the admitted pages (all KV heads, P x d 16-bit values each): block
// (i, 0) copies V of pair i, block (i, 1) its K; blocks past the plan's count exit.
__global__ __launch_bounds__(256) void hot_admit_copy_kernel(const uint16_t* __restrict__ v16,
                                                             uint16_t* __restrict__ v_hot,
                                                             const uint16_t* __restrict__ k16,
                                                             uint16_t* __restrict__ k_hot, size_t page_elems,
                                                             const int32_t* __restrict__ ws) {
  const int i = blockIdx.x;
  if (i >= ws[0]) return;
  const int p = ws[1 + 2 * i], s = ws[2 + 2 * i];
  const bool is_k = blockIdx.y == 1;
  const u32x4_t* src = reinterpret_cast<const u32x4_t*>((is_k ? k16 : v16) + (size_t)p * page_elems);
  u32x4_t* dst = reinterpret_cast<u32x4_t*>((is_k ? k_hot : v_hot) + (size_t)s * page_elems);
  const size_t n16 = page_elems / 8;
  for (size_t j = threadIdx.x; j < n16; j += 256) dst[j] = src[j];
}

hipError_t launch_hot_admit(const kv_layout& L, const void* v16, void* v_hot, const void* k16, void* k_hot,
                            int32_t* hot, int n_phys,
                            int32_t* slot_page, uint32_t* slot_stamp, int n_slots, const int32_t* block_table,
                            const int32_t* seq_lens, int B, int max_pages, const int32_t* sel,
                            const int32_t* sel_count, int k_max, uint32_t step, int32_t* ws, hipStream_t st) {
  const size_t lds = ((size_t)((n_phys + 31) >> 5) + (size_t)n_slots) * sizeof(uint32_t);
  hipError_t e = hipFuncSetAttribute((const void*)hot_admit_plan_kernel,
                                     hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(hot_admit_plan_kernel, dim3(1), dim3(kAdmitThreads), lds, st, block_table, seq_lens, B,
                     L.num_kv_heads, L.page_size, max_pages, sel, sel_count, k_max, hot, n_phys, slot_page,
                     slot_stamp, n_slots, step, ws);
  e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t page_elems = (size_t)L.num_kv_heads * L.page_size * L.head_dim;
  hipLaunchKernelGGL(hot_admit_copy_kernel, dim3(n_slots, k_hot ? 2 : 1), dim3(256), 0, st, (const uint16_t*)v16,
                     (uint16_t*)v_hot, (const uint16_t*)k16, (uint16_t*)k_hot, page_elems, ws);
  return hipGetLastError();
}

}  // namespace kvs
