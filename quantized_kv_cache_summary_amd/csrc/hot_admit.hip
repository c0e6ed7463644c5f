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
// The plan runs across the GPU as a chain of short kernels (no kernel waits
// on another's blocks):
//   clear    the unit bitmap;
//   mark     U into the bitmap (one thread per selection entry, atomic OR,
//            so duplicates vanish);
//   hits     one thread per bitmap word: hits stamp their slot, the word
//            keeps its misses, each block counts them;
//   plan     one block: scan of the block counts (each block's first miss),
//            the victim keys 0xFF7FFFFF - stamp of the slots stamped below the
//            step, n = min(misses, such slots), and the n-th largest key T with
//            how many keys equal to T are taken (the top-k selector's radix
//            search; ties by slot index);
//   misses   one thread per word: the misses, ascending, at their rank;
//   vcount   one thread per slot: per block, victims above T and equal to T;
//   vscan    one block: scans of those counts;
//   pair     one thread per slot: the victim of rank i takes the i-th miss.
// Then a copy kernel moves the admitted units.

#include "device.h"
#include "launch.h"
#include "select.h"

namespace kvs {

constexpr int kAdmitThreads = 1024;   // the one-block steps
constexpr int kAdmitBlock = 256;      // the grid-wide steps

// Exclusive prefix of v over a 256-thread block and the block total.
__device__ __forceinline__ int block_excl_scan_256(int v, int* wave_tot, int& total) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int incl = wave_incl_sum(v);
  if (lane == 63) wave_tot[wave] = incl;
  __syncthreads();
  int before = incl - v;
  total = 0;
#pragma unroll
  for (int w = 0; w < kAdmitBlock / 64; ++w) {
    if (w < wave) before += wave_tot[w];
    total += wave_tot[w];
  }
  return before;
}

__global__ __launch_bounds__(kAdmitBlock) void admit_clear_kernel(uint32_t* __restrict__ bits, int n_words) {
  const int w = blockIdx.x * kAdmitBlock + threadIdx.x;
  if (w < n_words) bits[w] = 0u;
}

__global__ __launch_bounds__(kAdmitBlock) void admit_mark_kernel(
    const int32_t* __restrict__ block_table, const int32_t* __restrict__ seq_lens, int Hkv, int P, int max_pages,
    const int32_t* __restrict__ sel, const int32_t* __restrict__ sel_count, int k_max, long long n_entries,
    int n_units, uint32_t* __restrict__ bits) {
  const long long e = (long long)blockIdx.x * kAdmitBlock + threadIdx.x;
  if (e >= n_entries) return;
  const int row = (int)(e / k_max), i = (int)(e - (long long)row * k_max);
  int cnt = sel_count[row];
  cnt = cnt < 0 ? 0 : (cnt > k_max ? k_max : cnt);
  if (i >= cnt) return;
  const int p = sel[e];
  const int b = row / Hkv, g = row - b * Hkv;
  const int L = seq_lens[b];
  int Np = L > 0 ? (L + P - 1) / P : 0;
  Np = Np < max_pages ? Np : max_pages;
  if (p < 0 || p >= Np) return;
  const int phys = block_table[(size_t)b * max_pages + p];
  const long long u = (long long)phys * Hkv + g;
  if (phys >= 0 && u < n_units) atomicOr(&bits[u >> 5], 1u << (u & 31));
}

__global__ __launch_bounds__(kAdmitBlock) void admit_hits_kernel(uint32_t* __restrict__ bits, int n_words,
                                                                 const int32_t* __restrict__ hot,
                                                                 uint32_t* __restrict__ slot_stamp, int n_slots,
                                                                 uint32_t step, int32_t* __restrict__ wcnt) {
  __shared__ int wave_tot[kAdmitBlock / 64];
  const int w = blockIdx.x * kAdmitBlock + threadIdx.x;
  uint32_t miss = 0u;
  if (w < n_words) {
    const uint32_t m = bits[w];
    if (m) {
      int hs[32];
#pragma unroll
      for (int j = 0; j < 32; ++j) hs[j] = (m >> j) & 1u ? hot[(w << 5) + j] : 0;
#pragma unroll
      for (int j = 0; j < 32; ++j) {
        if (!((m >> j) & 1u)) continue;
        const int sl = hs[j];
        if (sl >= 0 && sl < n_slots) slot_stamp[sl] = step;
        else miss |= 1u << j;
      }
      bits[w] = miss;
    }
  }
  int total;
  block_excl_scan_256(__popc(miss), wave_tot, total);
  if (threadIdx.x == 0) wcnt[blockIdx.x] = total;
}

// One block: miss offsets per word block, victim keys, n, the threshold.
// scal: [0] T, [1] take, [2] total misses.
__global__ __launch_bounds__(kAdmitThreads) void admit_plan_kernel(int32_t* __restrict__ wcnt, int n_wblocks,
                                                                   const uint32_t* __restrict__ slot_stamp,
                                                                   int n_slots, uint32_t step,
                                                                   uint32_t* __restrict__ keys,
                                                                   int32_t* __restrict__ ws,
                                                                   int32_t* __restrict__ scal) {
  constexpr int NT = kAdmitThreads;
  constexpr int NW = NT / 64;
  __shared__ SelectLds<NT> sh;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  if (tid == 0) sh.n_cand = 0;
  if (tid < kDirectMax) sh.cand[tid] = 0u;
  if (tid < 256) sh.hist[0][tid] = 0;

  // exclusive scan of the per-block miss counts, in place, chunk by chunk
  int carry = 0;
  for (int c0 = 0; c0 < n_wblocks; c0 += NT) {
    const int v = c0 + tid < n_wblocks ? wcnt[c0 + tid] : 0;
    const int incl = wave_incl_sum(v);
    if (lane == 63) sh.wave_tot[wave] = incl;
    __syncthreads();
    int before = incl - v, tot = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) before += sh.wave_tot[w];
      tot += sh.wave_tot[w];
    }
    if (c0 + tid < n_wblocks) wcnt[c0 + tid] = carry + before;
    carry += tot;
    __syncthreads();
  }
  const int total = carry;

  // victim keys: larger key = older; slots stamped at this step take -inf
  int n_free = 0;
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  constexpr int kSlots = 8;
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
  uint32_t T = 0xFFFFFFFFu;   // no victim
  int take = 0;
  if (n > 0) select_kth<NT>(sh, keys, n_slots, st, n, T, take);
  if (tid == 0) {
    ws[0] = n;
    scal[0] = (int32_t)T;
    scal[1] = take;
    scal[2] = total;
  }
}

// The misses of each word at their rank in ascending unit order (the first
// n_slots of them).
__global__ __launch_bounds__(kAdmitBlock) void admit_misses_kernel(const uint32_t* __restrict__ bits, int n_words,
                                                                   const int32_t* __restrict__ woff, int n_slots,
                                                                   int32_t* __restrict__ miss) {
  __shared__ int wave_tot[kAdmitBlock / 64];
  const int w = blockIdx.x * kAdmitBlock + threadIdx.x;
  uint32_t m = w < n_words ? bits[w] : 0u;
  int total;
  int pos = woff[blockIdx.x] + block_excl_scan_256(__popc(m), wave_tot, total);
  while (m && pos < n_slots) {
    const int bit = __ffs((int)m) - 1;
    m &= m - 1u;
    miss[pos++] = (w << 5) + bit;
  }
}

// Per slot block: victims with key above T and equal to T.
__global__ __launch_bounds__(kAdmitBlock) void admit_vcount_kernel(const uint32_t* __restrict__ keys, int n_slots,
                                                                   const int32_t* __restrict__ ws,
                                                                   const int32_t* __restrict__ scal,
                                                                   int32_t* __restrict__ vcnt) {
  __shared__ int wave_tot[kAdmitBlock / 64];
  if (ws[0] == 0) return;   // uniform: nothing admitted
  const uint32_t T = (uint32_t)scal[0];
  const int s = blockIdx.x * kAdmitBlock + threadIdx.x;
  const uint32_t key = s < n_slots ? keys[s] : 0u;
  int tg, te;
  block_excl_scan_256(key > T, wave_tot, tg);
  __syncthreads();
  block_excl_scan_256(key == T, wave_tot, te);
  if (threadIdx.x == 0) {
    vcnt[2 * blockIdx.x] = tg;
    vcnt[2 * blockIdx.x + 1] = te;
  }
}

// One block: exclusive scans of the (above, equal) counts, in place.
__global__ __launch_bounds__(kAdmitThreads) void admit_vscan_kernel(int32_t* __restrict__ vcnt, int n_sblocks,
                                                                    const int32_t* __restrict__ ws) {
  constexpr int NT = kAdmitThreads;
  constexpr int NW = NT / 64;
  __shared__ int tot_g[NW], tot_e[NW];
  if (ws[0] == 0) return;
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  int carry_g = 0, carry_e = 0;
  for (int c0 = 0; c0 < n_sblocks; c0 += NT) {
    const int i = c0 + tid;
    const int g = i < n_sblocks ? vcnt[2 * i] : 0, e = i < n_sblocks ? vcnt[2 * i + 1] : 0;
    const int ig = wave_incl_sum(g), ie = wave_incl_sum(e);
    if (lane == 63) { tot_g[wave] = ig; tot_e[wave] = ie; }
    __syncthreads();
    int bg = ig - g, be = ie - e, sg = 0, se = 0;
#pragma unroll
    for (int w = 0; w < NW; ++w) {
      if (w < wave) { bg += tot_g[w]; be += tot_e[w]; }
      sg += tot_g[w];
      se += tot_e[w];
    }
    if (i < n_sblocks) { vcnt[2 * i] = carry_g + bg; vcnt[2 * i + 1] = carry_e + be; }
    carry_g += sg;
    carry_e += se;
    __syncthreads();
  }
}

// The victim of rank i (ascending slot) takes the i-th miss.  A victim's old
// unit was not called this step, so it is none of the misses: the stores of
// different slots never meet.
__global__ __launch_bounds__(kAdmitBlock) void admit_pair_kernel(const uint32_t* __restrict__ keys, int n_slots,
                                                                 const int32_t* __restrict__ vcnt,
                                                                 const int32_t* __restrict__ scal,
                                                                 const int32_t* __restrict__ miss,
                                                                 int32_t* __restrict__ hot, int n_units,
                                                                 int32_t* __restrict__ slot_page,
                                                                 uint32_t* __restrict__ slot_stamp, uint32_t step,
                                                                 int32_t* __restrict__ ws) {
  __shared__ int wave_tot[kAdmitBlock / 64];
  const int n = ws[0];
  if (n == 0) return;
  const uint32_t T = (uint32_t)scal[0];
  const int take = scal[1];
  const int s = blockIdx.x * kAdmitBlock + threadIdx.x;
  const uint32_t key = s < n_slots ? keys[s] : 0u;
  int tg, te;
  const int gb = vcnt[2 * blockIdx.x] + block_excl_scan_256(key > T, wave_tot, tg);
  __syncthreads();
  const int eb = vcnt[2 * blockIdx.x + 1] + block_excl_scan_256(key == T, wave_tot, te);
  if (s >= n_slots) return;
  if (!(key > T || (key == T && eb < take))) return;
  const int i = gb + (eb < take ? eb : take);
  if (i >= n) return;
  const int p = miss[i];
  if (p < 0 || p >= n_units) return;   // never, for a plan of this call
  const int old = slot_page[s];
  if (old >= 0 && old < n_units) hot[old] = -1;
  slot_page[s] = p;
  hot[p] = s;
  slot_stamp[s] = step;
  ws[1 + 2 * i] = p;
  ws[2 + 2 * i] = s;
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
  int32_t* wcnt = ws + lay.wcnt;
  int32_t* vcnt = ws + lay.vcnt;
  int32_t* scal = ws + lay.scal;
  int32_t* miss = ws + 1 + 2 * (size_t)n_slots;
  const int Hkv = L.num_kv_heads;
  const int n_words = (n_units + 31) >> 5;
  const int n_wblocks = (n_words + kAdmitBlock - 1) / kAdmitBlock;
  const int n_sblocks = (n_slots + kAdmitBlock - 1) / kAdmitBlock;
  const long long n_entries = (long long)B * Hkv * k_max;
  const dim3 blk(kAdmitBlock);
  hipLaunchKernelGGL(admit_clear_kernel, dim3(n_wblocks), blk, 0, st, bits, n_words);
  if (n_entries > 0)
    hipLaunchKernelGGL(admit_mark_kernel, dim3((unsigned)((n_entries + kAdmitBlock - 1) / kAdmitBlock)), blk, 0, st,
                       block_table, seq_lens, Hkv, L.page_size, max_pages, sel, sel_count, k_max, n_entries,
                       n_units, bits);
  hipLaunchKernelGGL(admit_hits_kernel, dim3(n_wblocks), blk, 0, st, bits, n_words, (const int32_t*)hot, slot_stamp,
                     n_slots, step, wcnt);
  hipLaunchKernelGGL(admit_plan_kernel, dim3(1), dim3(kAdmitThreads), 0, st, wcnt, n_wblocks,
                     (const uint32_t*)slot_stamp, n_slots, step, keys, ws, scal);
  hipLaunchKernelGGL(admit_misses_kernel, dim3(n_wblocks), blk, 0, st, (const uint32_t*)bits, n_words,
                     (const int32_t*)wcnt, n_slots, miss);
  hipLaunchKernelGGL(admit_vcount_kernel, dim3(n_sblocks), blk, 0, st, (const uint32_t*)keys, n_slots,
                     (const int32_t*)ws, (const int32_t*)scal, vcnt);
  hipLaunchKernelGGL(admit_vscan_kernel, dim3(1), dim3(kAdmitThreads), 0, st, vcnt, n_sblocks, (const int32_t*)ws);
  hipLaunchKernelGGL(admit_pair_kernel, dim3(n_sblocks), blk, 0, st, (const uint32_t*)keys, n_slots,
                     (const int32_t*)vcnt, (const int32_t*)scal, (const int32_t*)miss, hot, n_units, slot_page,
                     slot_stamp, step, ws);
  hipError_t e = hipGetLastError();
  if (e != hipSuccess) return e;
  const size_t unit_elems = (size_t)L.page_size * L.head_dim;
  const int grid = n_slots < 2048 ? n_slots : 2048;
  hipLaunchKernelGGL(hot_admit_copy_kernel, dim3(grid, k_hot ? 2 : 1), dim3(256), 0, st, (const uint16_t*)v16,
                     (uint16_t*)v_hot, (const uint16_t*)k16, (uint16_t*)k_hot, unit_elems, n_units, n_slots, ws);
  return hipGetLastError();
}

}  // namespace kvs
