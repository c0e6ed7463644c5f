// Hot-buffer admission for a host-resident value pool.  AMASS (amass-kv 0.1.1
// project page), "What is in the box" item 2 and the AMASS-mem variant: V in
// pinned, device-mapped host memory with a bounded resident hot buffer and a
// staging pool; only the pages a step calls stay in device memory.
//
// The buffer's unit is one (physical page, KV head), u = phys * Hkv + g: the
// P x d values one row's attention reads of a page.  Once per step, after its
// selection and before its attention, with U = the units the step's
// selections name (entries i < sel_count of row (b, g), pages p < Np_b,
// through the block table), with no duplicates:
//   1. a unit of U already hot has its slot stamped with the step;
//   2. the units of U not hot, ascending by unit id, go to the slots least
//      recently used before this step (smallest (stamp, slot index) among
//      slots stamped below the step), one per slot, paired in ascending slot
//      order; with fewer such slots than units, the lowest unit ids win;
//   3. an admitted slot drops its old unit, takes the new one, is stamped, and
//      the unit's V is copied in from the pool; with a K hot buffer (the
//      mem-kv variant: K offloaded as well) its K too.
// The attention that follows reads every admitted unit from device memory, so
// a called unit crosses the host link once.
//
// One block plans the step: U as a bitmap in the workspace (integer atomics),
// the misses by an ordered compaction of the bitmap, the victim slots as the
// k largest of the keys 0xFF7FFFFF - stamp with the selector's radix search
// and ordered compaction (ties by slot index).  A second kernel copies the
// admitted units.

#include "device.h"
#include "launch.h"
#include "select.h"

namespace kvs {

constexpr int kAdmitThreads = 1024;

// Workspace (int32 words): [0] number of copies, (unit, slot) pairs
// [1, 1 + 2 n_slots), the miss list [1 + 2 n_slots, 1 + 3 n_slots), then the
// unit bitmap and the slot keys at 64-word boundaries (hot_admit_ws_layout).
__global__ __launch_bounds__(kAdmitThreads) void hot_admit_plan_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int B, int Hkv, int P,
    int max_pages, const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int k_max,
    int32_t* __restrict__ hot, int n_units, int32_t* __restrict__ slot_page, uint32_t* __restrict__ slot_stamp,
    int n_slots, uint32_t step, int32_t* __restrict__ ws, uint32_t* __restrict__ bits,
    uint32_t* __restrict__ keys) {
  constexpr int NT = kAdmitThreads;
  constexpr int NW = NT / 64;
  const int n_words = (n_units + 31) >> 5;
  __shared__ SelectLds<NT> sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  for (int w = tid; w < n_words; w += NT) bits[w] = 0u;
  if (tid == 0) sh.n_cand = 0;
  if (tid < kDirectMax) sh.cand[tid] = 0u;
  if (tid < 256) sh.hist[0][tid] = 0;
  __syncthreads();

  // 1. U: every valid selection entry, through the block table, as the unit
  //    phys * Hkv + g of its row's KV head g; a thread takes kBatch entries at
  //    a time so their loads are in flight together
  constexpr int kBatch = 16;
  const size_t n_entries = (size_t)B * Hkv * k_max;
  for (size_t e0 = tid; e0 < n_entries; e0 += (size_t)NT * kBatch) {
    int p[kBatch], b[kBatch], g[kBatch];
#pragma unroll
    for (int j = 0; j < kBatch; ++j) {
      const size_t e = e0 + (size_t)j * NT;
      p[j] = -1;
      b[j] = 0;
      g[j] = 0;
      if (e < n_entries) {
        const int row = (int)(e / k_max), i = (int)(e - (size_t)row * k_max);
        int cnt = sel_count[row];
        cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
        b[j] = row / Hkv;
        g[j] = row - b[j] * Hkv;
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
    for (int j = 0; j < kBatch; ++j) {
      const long long u = (long long)p[j] * Hkv + g[j];
      if (p[j] >= 0 && u < n_units) atomicOr(&bits[u >> 5], 1u << (u & 31));
    }
  }
  __syncthreads();

  // 2. hits get the step's stamp; each word of the bitmap is replaced by its
  //    misses (the hot-map loads of a word are in flight together), then the
  //    misses are listed ascending (each thread owns a contiguous run of
  //    words).  The words were set by device-scope atomics: read them past
  //    the first-level cache.
  const int chunk = (n_words + NT - 1) / NT;
  const int w0 = tid * chunk, w1 = w0 + chunk < n_words ? w0 + chunk : n_words;
  int my_miss = 0;
  constexpr int kWords = 8;   // words whose loads are in flight together
  for (int wb = w0; wb < w1; wb += kWords) {
    uint32_t mw[kWords];
#pragma unroll
    for (int q = 0; q < kWords; ++q)
      mw[q] = wb + q < w1 ? __hip_atomic_load(&bits[wb + q], __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) : 0u;
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
      const uint32_t m = mw[q];
      if (m == 0u) continue;
      const int w = wb + q;
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
  int32_t* miss = ws + 1 + 2 * (size_t)n_slots;   // the first n_slots misses, ascending
  int pos = before;
  for (int wb = w0; wb < w1 && pos < n_slots; wb += kWords) {
    uint32_t mw[kWords];
#pragma unroll
    for (int q = 0; q < kWords; ++q) mw[q] = wb + q < w1 ? bits[wb + q] : 0u;
#pragma unroll
    for (int q = 0; q < kWords; ++q) {
      uint32_t m = mw[q];
      while (m && pos < n_slots) {
        const int bit = __ffs((int)m) - 1;
        m &= m - 1u;
        miss[pos++] = ((wb + q) << 5) + bit;
      }
    }
  }
  __syncthreads();   // hit stamps and the miss list are visible to the block

  // 3. victim slots: keys 0xFF7FFFFF - stamp for slots stamped below the step
  //    (larger key = older), the others at the -inf key
  int n_free = 0;
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  constexpr int kSlots = 8;   // slots whose stamps are in flight together
  for (int s0 = tid; s0 < n_slots; s0 += NT * kSlots) {
    uint32_t sv[kSlots];
#pragma unroll
    for (int q = 0; q < kSlots; ++q) sv[q] = s0 + q * NT < n_slots ? slot_stamp[s0 + q * NT] : step;
#pragma unroll
    for (int q = 0; q < kSlots; ++q) {
      const int s = s0 + q * NT;
      if (s >= n_slots) break;
      const uint32_t st = sv[q];
      uint32_t key = kKeyNegInf;
      if (st < step) {
        key = 0xFF7FFFFFu - (st < 0xFEFFFFFFu ? st : 0xFEFFFFFFu);
        ++n_free;
        kmax = key > kmax ? key : kmax;
        kmin = key < kmin ? key : kmin;
      }
      keys[s] = key;
    }
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

  // 4. the i-th victim in ascending slot order goes to ws[2 + 2i]; then the
  //    i-th victim takes the i-th miss (ascending unit).  A victim's old unit
  //    was not called this step, so it is none of the misses: the stores of
  //    different pairs never meet.
  select_compact<NT, true>(sh, keys, n_slots, T, take, [&](int s, int i) {
    if (i < n) ws[2 + 2 * i] = s;
  });
  __syncthreads();
  constexpr int kPairs = 8;   // pairs whose loads are in flight together
  for (int i0 = tid; i0 < n; i0 += NT * kPairs) {
    int sv[kPairs], pv[kPairs], ov[kPairs];
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      const int i = i0 + q * NT;
      sv[q] = i < n ? ws[2 + 2 * i] : 0;
      pv[q] = i < n ? miss[i] : 0;
    }
    // every position i < n was written above; the range checks only keep a
    // broken plan in bounds
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      const bool ok = i0 + q * NT < n && sv[q] >= 0 && sv[q] < n_slots && pv[q] >= 0 && pv[q] < n_units;
      ov[q] = ok ? slot_page[sv[q]] : -2;
    }
#pragma unroll
    for (int q = 0; q < kPairs; ++q) {
      const int i = i0 + q * NT;
      if (i >= n) break;
      if (ov[q] == -2) continue;
      if (ov[q] >= 0 && ov[q] < n_units) hot[ov[q]] = -1;
      slot_page[sv[q]] = pv[q];
      hot[pv[q]] = sv[q];
      slot_stamp[sv[q]] = step;
      ws[1 + 2 * i] = pv[q];
    }
  }
}

// Copies the admitted units (P x d 16-bit values each): blocks stride over the
// plan's pairs, blockIdx.y = 0 for V, 1 for K.
__global__ __launch_bounds__(256) void hot_admit_copy_kernel(const uint16_t* __restrict__ v16,
                                                             uint16_t* __restrict__ v_hot,
                                                             const uint16_t* __restrict__ k16,
                                                             uint16_t* __restrict__ k_hot, size_t unit_elems,
                                                             int n_units, int n_slots,
                                                             const int32_t* __restrict__ ws) {
  int n = ws[0];
  n = n < n_slots ? n : n_slots;
  const bool is_k = blockIdx.y == 1;
  const uint16_t* pool = is_k ? k16 : v16;
  uint16_t* buf = is_k ? k_hot : v_hot;
  const size_t n16 = unit_elems / 8;
  for (int i = blockIdx.x; i < n; i += gridDim.x) {
    const int u = ws[1 + 2 * i], s = ws[2 + 2 * i];
    if (u < 0 || u >= n_units || s < 0 || s >= n_slots) continue;   // never, for a plan of this call
    const u32x4_t* src = reinterpret_cast<const u32x4_t*>(pool + (size_t)u * unit_elems);
    u32x4_t* dst = reinterpret_cast<u32x4_t*>(buf + (size_t)s * unit_elems);
    for (size_t j = threadIdx.x; j < n16; j += 256) dst[j] = src[j];
  }
}

hipError_t launch_hot_admit(const kv_layout& L, const void* v16, void* v_hot, const void* k16, void* k_hot,
                            int32_t* hot, int n_units,
                            int32_t* slot_page, uint32_t* slot_stamp, int n_slots, const int32_t* block_table,
                            const int32_t* seq_lens, int B, int max_pages, const int32_t* sel,
                            const int32_t* sel_count, int k_max, uint32_t step, int32_t* ws, hipStream_t st) {
  const HotAdmitWs lay = hot_admit_ws_layout(n_slots, n_units);
  uint32_t* bits = reinterpret_cast<uint32_t*>(ws + lay.bits);
  uint32_t* keys = reinterpret_cast<uint32_t*>(ws + lay.keys);
  hipLaunchKernelGGL(hot_admit_plan_kernel, dim3(1), dim3(kAdmitThreads), 0, st, block_table, seq_lens, B,
                     L.num_kv_heads, L.page_size, max_pages, sel, sel_count, k_max, hot, n_units, slot_page,
                     slot_stamp, n_slots, step, ws, bits, keys);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t unit_elems = (size_t)L.page_size * L.head_dim;
  const int grid = n_slots < 2048 ? n_slots : 2048;
  hipLaunchKernelGGL(hot_admit_copy_kernel, dim3(grid, k_hot ? 2 : 1), dim3(256), 0, st, (const uint16_t*)v16,
                     (uint16_t*)v_hot, (const uint16_t*)k16, (uint16_t*)k_hot, unit_elems, n_units, n_slots, ws);
  return hipGetLastError();
}

}  // namespace kvs
