// Exact top-k page selection for one (sequence, KV head) row, by one block of
// NT threads.  AMASS (amass-kv 0.1.1 project page), "Quickstart" (budget: a
// fixed selected page fraction) and "Benchmarking" (the top-B stage).
//
//   L_h = logsumexp_p s[h][p]                 (merged from the score blocks'
//                                              (max, sum exp) partials)
//   S_p = log((1/G) sum_h exp(s[h][p] - L_h))  (group-mean mass fraction)
//
// The k-th largest S is found exactly on order-preserving uint32 keys.  The
// +inf keys (forced pages) and -inf keys (empty or NaN scores) are counted
// apart, so the radix passes start at the highest bit in which the row's
// finite keys differ: scores of one row share sign and most exponent bits,
// and a digit taken above that would put nearly every key in one bin.  Each
// pass is an 8-bit LDS histogram with integer counts (independent of thread
// timing); once the bin holding the k-th key has at most kDirectMax keys they
// are ranked against each other directly instead of by further passes.  An
// ordered compaction then keeps every key above the threshold and the
// lowest-index pages among keys equal to it, so pages come out ascending with
// no sort and ties break by (S descending, page ascending) exactly.
#pragma once

#include "device.h"

namespace kvs {

constexpr uint32_t kKeyNegInf = 0x007FFFFFu;   // key of -inf; NaN scores take it too
constexpr uint32_t kKeyPosInf = 0xFF800000u;   // key of +inf (forced pages)
constexpr int kDirectMax = 64;                  // bin size finished by direct ranking

__device__ __forceinline__ uint32_t order_key(float S) {
  if (S != S) return kKeyNegInf;
  S = S + 0.0f;   // -0 -> +0
  const uint32_t u = __float_as_uint(S);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ bool finite_key(uint32_t key) { return key > kKeyNegInf && key < kKeyPosInf; }

// Pages kept for a row of Np pages: k_fixed if set, else ceil(keep * Np), in [1, Np].
__device__ __forceinline__ int selection_count(int Np, float keep, int k_fixed) {
  if (Np <= 0) return 0;
  if (k_fixed > 0) return k_fixed < Np ? k_fixed : Np;
  int k = (int)ceil((double)keep * (double)Np);
  return k < 1 ? 1 : (k > Np ? Np : k);
}

template <int NT>
struct SelectLds {
  static_assert(NT >= 256 && NT % 64 == 0, "every lane scans four of the 256 bins");
  static constexpr int NW = NT / 64;
  float Lh[16];
  int hist[3][256];   // three buffers: one pass fills one, clears the next, reads back the one it filled
  int wave_tot[NW];
  uint32_t wmax[NW], wmin[NW];
  int wpos[NW], wneg[NW];
  alignas(16) uint32_t cand[kDirectMax];
  int n_cand;
  // coverage mode: per-bin masses in fixed point, forced pages' mass
  unsigned long long hmass[3][256];
  unsigned long long forced_mass;
};

// Row statistics of the keys (block-uniform).
struct SelectStats {
  uint32_t kmax, kmin;   // extremes of the finite keys
  int npos, nneg;        // +inf keys (forced pages), -inf keys (empty or NaN)
};

// Page mass exp(S) in fixed point with 40 fraction bits (S <= 0 for a
// log-distribution; larger values clamp at 1).  Integer sums are exact, so the
// coverage count does not depend on the order of accumulation.
constexpr float kMassScale = 1099511627776.0f;   // 2^40
__device__ __forceinline__ unsigned long long mass_fixed(float S) {
  if (!(S == S)) return 0ull;
  const float m = fminf(__expf(S), 1.0f);
  return (unsigned long long)(m * kMassScale);
}
__device__ __forceinline__ float key_to_score(uint32_t key) {
  return __uint_as_float((key & 0x80000000u) ? (key & 0x7FFFFFFFu) : ~key);
}

// Register-held inputs: the first round of head scores (U pages per thread,
// strided by NT) and the score blocks' (max, sum exp) partials of the heads
// this wave normalises (tiles lane + 64 i).
template <int NT, int GM>
struct SelectLoads {
  static constexpr int NW = NT / 64;
  // pages per thread per round: 2048 pages per round for blocks under 1024
  // threads (the fused kernel's register budget); the 1024-thread selector of
  // long rows keeps up to 64 scores per thread in flight (4096 pages a round
  // at up to eight heads), so a 4096-page row is one round and an 8192-page
  // row two
  static constexpr int U0 = (NT >= 1024 ? 4096 : 2048) / NT, U1 = (NT >= 1024 && GM <= 8 ? 64 : 32) / GM;
  static constexpr int U = U0 < U1 ? U0 : U1;
  static constexpr int HJ = (GM + NW - 1) / NW;
  static constexpr int TI = 4;   // up to 256 score tiles per row
  float v[U][GM];
  float2 part[HJ][TI];
};

template <int NT, int GM, int U>
__device__ __forceinline__ void select_load_round(float (&v)[U][GM], const float* hs, int G, int max_pages,
                                                  int p0) {
#pragma unroll
  for (int u = 0; u < U; ++u) {
    const int p = p0 + u * NT;
    const int pc = p < max_pages ? p : max_pages - 1;   // in bounds; values past the row are ignored
#pragma unroll
    for (int h = 0; h < GM; ++h) v[u][h] = hs[(size_t)(h < G ? h : 0) * max_pages + pc];
  }
}

// Requests every input the threshold search starts from.  No address depends
// on the row length, so the loads leave before it is known.  hs: the row's
// [G][max_pages] head scores; lsep: its [n_tiles][G] partial pairs.
// max_pages >= 1, n_tiles <= 256.
template <int NT, int GM>
__device__ __forceinline__ void select_issue(SelectLoads<NT, GM>& ld, const float* hs, const float* lsep,
                                             int G, int max_pages, int n_tiles) {
  using SL = SelectLoads<NT, GM>;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  select_load_round<NT, GM>(ld.v, hs, G, max_pages, threadIdx.x);
#pragma unroll
  for (int j = 0; j < SL::HJ; ++j) {
    const int h = wave + SL::NW * j;
    const int hc = h < G ? h : 0;
#pragma unroll
    for (int i = 0; i < SL::TI; ++i) {
      if (64 * i < n_tiles) {
        const int t = lane + 64 * i < n_tiles ? lane + 64 * i : n_tiles - 1;
        ld.part[j][i] = *reinterpret_cast<const float2*>(lsep + ((size_t)t * G + hc) * 2);
      }
    }
  }
}

// Calls f(key) for the keys of pages [0, Np) this thread owns (p = tid + j NT).
// Reads are issued KB at a time before any is used, so a pass costs a few LDS
// round trips rather than one per key.
template <int NT, typename F>
__device__ __forceinline__ void for_own_keys(const uint32_t* keys, int Np, F&& f) {
  constexpr int KB = 4;
  for (int p0 = threadIdx.x; p0 < Np; p0 += KB * NT) {
    uint32_t kv[KB];
#pragma unroll
    for (int i = 0; i < KB; ++i) kv[i] = p0 + i * NT < Np ? keys[p0 + i * NT] : kKeyNegInf;
#pragma unroll
    for (int i = 0; i < KB; ++i) f(kv[i]);
  }
}

// Threshold of the row: the k-th largest key T and how many keys equal to T
// are kept (the lowest-index ones).  Leaves the keys of pages [0, Np) in
// keys[].  select_issue must have been called.  k >= 1.  Block-uniform results.
// Keys of pages [0, Np) into keys[] and their statistics.  select_issue must
// have been called.  With with_mass, the forced pages' own masses (before their
// score is raised to +inf) are summed into sh.forced_mass.
template <int NT, int GM>
__device__ SelectStats select_keys(SelectLds<NT>& sh, uint32_t* keys, SelectLoads<NT, GM>& ld,
                                   const float* hs, int G, int max_pages, int n_tiles, int Np,
                                   int n_force_first, int n_force_last, float* page_S_row, bool with_mass) {
  using SL = SelectLoads<NT, GM>;
  constexpr int NW = NT / 64;
  constexpr int U = SL::U;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);

  // 1. per-head normalisers L_h from the partials
#pragma unroll
  for (int j = 0; j < SL::HJ; ++j) {
    const int h = wave + NW * j;
    if (h < G) {
      float m = -INFINITY, s = 0.f;
#pragma unroll
      for (int i = 0; i < SL::TI; ++i)
        if (64 * i < n_tiles && lane + 64 * i < n_tiles) lse_merge(m, s, ld.part[j][i].x, ld.part[j][i].y);
      const float M = wave_max_f32(m);
      const float S = wave_sum_f32(m == -INFINITY ? 0.f : s * __expf(m - M));
      if (lane == 0) sh.Lh[h] = (S > 0.f || S != S) ? M + __logf(S) : -INFINITY;
    }
  }
  if (tid == 0) { sh.n_cand = 0; sh.forced_mass = 0ull; }
  if (tid < kDirectMax) sh.cand[tid] = 0u;   // below every finite key
  if (tid < 256) { sh.hist[0][tid] = 0; sh.hmass[0][tid] = 0ull; }
  __syncthreads();

  // 2. group aggregate and keys, the next round of scores in flight while one
  //    is reduced; extremes of the finite keys, counts of the infinite ones
  const float logG = __logf((float)G);
  float Lr[GM];
#pragma unroll
  for (int h = 0; h < GM; ++h) Lr[h] = h < G ? sh.Lh[h] : 0.f;
  uint32_t kmax = 0u, kmin = 0xFFFFFFFFu;
  int npos = 0, nneg = 0;
  unsigned long long fmass = 0ull;
  // Straight-line per page (selects, no branches): head slots past G enter as
  // -inf, whose exp is an exact +0 at the end of the sum, so S is the same as
  // over the G heads alone; NaN and all -inf rows are patched in afterwards.
  for (int r0 = 0; r0 < Np; r0 += NT * U) {
    const bool more = r0 + NT * U < Np;
    float nx[U][GM];
    if (more) select_load_round<NT, GM>(nx, hs, G, max_pages, r0 + NT * U + tid);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int p = r0 + tid + u * NT;
      const bool live = p < Np;
      float x[GM];
      float M = -INFINITY;
      bool nan = false;
#pragma unroll
      for (int h = 0; h < GM; ++h) {
        x[h] = h < G ? ld.v[u][h] - Lr[h] : -INFINITY;
        nan |= x[h] != x[h];
        M = fmaxf(M, x[h]);
      }
      float sum = 0.f;
#pragma unroll
      for (int h = 0; h < GM; ++h) sum += __expf(x[h] - M);
      float S = M + __logf(sum) - logG;
      S = M == -INFINITY ? -INFINITY : S;
      S = nan ? __int_as_float(0x7FC00000) : S;
      const bool forced = p < n_force_first || p >= Np - n_force_last;
      if (with_mass && live && forced) fmass += mass_fixed(S);
      S = forced ? INFINITY : S;
      const uint32_t key = order_key(S);
      if (live) {
        keys[p] = key;
        if (page_S_row) page_S_row[p] = S;
      }
      const bool fin = live && finite_key(key);
      kmax = fin && key > kmax ? key : kmax;
      kmin = fin && key < kmin ? key : kmin;
      npos += live && key == kKeyPosInf;
      nneg += live && key == kKeyNegInf;
    }
    if (more) {
#pragma unroll
      for (int u = 0; u < U; ++u)
#pragma unroll
        for (int h = 0; h < GM; ++h) ld.v[u][h] = nx[u][h];
    }
  }
  if (with_mass && fmass) atomicAdd(&sh.forced_mass, fmass);
  kmax = wave_max_u32(kmax);
  kmin = wave_min_u32(kmin);
  const int pn = wave_sum_i32((npos << 16) | nneg);   // both counts < 2^15: one packed sum
  if (lane == 0) { sh.wmax[wave] = kmax; sh.wmin[wave] = kmin; sh.wpos[wave] = pn >> 16; sh.wneg[wave] = pn & 0xFFFF; }
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
  return st;
}

// Threshold of the row: the k-th largest key T and how many keys equal to T
// are kept (the lowest-index ones).  1 <= k <= Np.  Block-uniform results.
template <int NT>
__device__ void select_kth(SelectLds<NT>& sh, const uint32_t* keys, int Np, const SelectStats& stt, int k,
                           uint32_t& T_out, int& take_out) {
  const int tid = threadIdx.x, lane = tid & 63;
  const uint32_t kmax = stt.kmax, kmin = stt.kmin;
  const int npos = stt.npos, nneg = stt.nneg;

  // 3. the k-th largest key
  int rem = k;
  if (rem <= npos) {                         // only forced (+inf) pages are kept
    T_out = kKeyPosInf;
    take_out = rem;
    return;
  }
  rem -= npos;
  const int nfin = Np - npos - nneg;
  if (rem > nfin) {                          // every finite page is kept, and some -inf ones
    T_out = kKeyNegInf;
    take_out = rem - nfin;
    return;
  }
  if (kmax == kmin) {                        // all finite keys equal
    T_out = kmax;
    take_out = rem;
    return;
  }
  const uint32_t diff = kmax ^ kmin;
  const int hb = 31 - __clz((int)diff);
  uint32_t pmask = hb >= 31 ? 0u : ~((2u << hb) - 1u);   // common prefix of the finite keys
  uint32_t prefix = kmax & pmask;
  int top = hb;                                          // highest bit of the next digit
  int buf = 0;
  for (;;) {
    const int width = top + 1 < 8 ? top + 1 : 8;
    const int shift = top + 1 - width;
    const uint32_t dmask = (1u << width) - 1u;
    for_own_keys<NT>(keys, Np, [&](uint32_t key) {
      if ((key & pmask) == prefix && finite_key(key)) atomicAdd(&sh.hist[buf][(key >> shift) & dmask], 1);
    });
    const int nb = buf == 2 ? 0 : buf + 1;
    if (tid < 256) sh.hist[nb][tid] = 0;
    __syncthreads();
    // every wave finds the digit itself, so no second barrier is needed:
    // lane l owns digits 255-4l .. 252-4l (descending); unused digits count 0
    int c[4], tot = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) { c[i] = sh.hist[buf][255 - 4 * lane - i]; tot += c[i]; }
    const int incl = wave_incl_sum(tot);
    const int first = __ffsll((long long)__ballot(incl >= rem)) - 1;
    int cum = incl - tot, dsel = 252 - 4 * lane, dcnt = c[3];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (cum + c[i] >= rem) { dsel = 255 - 4 * lane - i; dcnt = c[i]; break; }
      cum += c[i];
    }
    dsel = __builtin_amdgcn_readlane(dsel, first);
    cum = __builtin_amdgcn_readlane(cum, first);
    dcnt = __builtin_amdgcn_readlane(dcnt, first);
    prefix |= (uint32_t)dsel << shift;
    pmask |= dmask << shift;
    rem -= cum;
    buf = nb;
    top -= width;
    if (top < 0) {                             // every bit fixed: T is the prefix
      T_out = prefix;
      take_out = rem;
      return;
    }
    if (dcnt <= kDirectMax) break;
  }

  // 4. direct finish: every wave ranks the (at most kDirectMax) keys left in the bin
  for_own_keys<NT>(keys, Np, [&](uint32_t key) {
    if ((key & pmask) == prefix && finite_key(key)) {
      const int slot = atomicAdd(&sh.n_cand, 1);
      if (slot < kDirectMax) sh.cand[slot] = key;
    }
  });
  __syncthreads();
  const int nc = sh.n_cand < kDirectMax ? sh.n_cand : kDirectMax;
  const uint32_t x = lane < nc ? sh.cand[lane] : 0u;
  int gt = 0, ge = 0;
  // four slots per read; unused slots hold 0, which no finite key is below
  for (int j = 0; j < nc; j += 4) {
    const uint4 y = *reinterpret_cast<const uint4*>(&sh.cand[j]);
    gt += (y.x > x) + (y.y > x) + (y.z > x) + (y.w > x);
    ge += (y.x >= x) + (y.y >= x) + (y.z >= x) + (y.w >= x);
  }
  const int first = __ffsll((long long)__ballot(lane < nc && gt < rem && rem <= ge)) - 1;
  T_out = (uint32_t)__builtin_amdgcn_readlane((int)x, first);
  take_out = rem - __builtin_amdgcn_readlane(gt, first);
}

// Keys and the threshold for a fixed k (>= 1).
template <int NT, int GM>
__device__ void select_threshold(SelectLds<NT>& sh, uint32_t* keys, SelectLoads<NT, GM>& ld,
                                 const float* hs, int G, int max_pages, int n_tiles, int Np, int k,
                                 int n_force_first, int n_force_last, float* page_S_row,
                                 uint32_t& T_out, int& take_out) {
  const SelectStats st = select_keys<NT, GM>(sh, keys, ld, hs, G, max_pages, n_tiles, Np, n_force_first,
                                             n_force_last, page_S_row, false);
  select_kth<NT>(sh, keys, Np, st, k, T_out, take_out);
}

// Coverage mode: the length of the shortest prefix of the selection order
// (forced pages first, then keys descending, equal keys by page) whose total
// mass exp(S) reaches `coverage` (forced pages with their own mass, -inf keys
// with none); every page if it is never reached.  Then clamped to
// [max(1, forced pages), min(k_cap, Np)].  The crossing is found by radix
// passes over the finite keys with per-bin counts and fixed-point masses; the
// keys equal to the final threshold share one mass, so the count needed among
// them is a division.  Block-uniform result.
template <int NT>
__device__ int select_coverage_k(SelectLds<NT>& sh, const uint32_t* keys, int Np, const SelectStats& stt,
                                 float coverage, int k_cap) {
  const int tid = threadIdx.x, lane = tid & 63;
  const int npos = stt.npos, nfin = Np - stt.npos - stt.nneg;
  int lo = npos > 1 ? npos : 1;
  int hi = k_cap < Np ? k_cap : Np;
  auto clampk = [&](int k) { k = k < lo ? lo : k; return k > hi ? hi : k; };
  if (!(coverage <= 1.0f)) return clampk(Np);               // never reached (or NaN coverage)
  const unsigned long long target = (unsigned long long)(fmaxf(coverage, 0.f) * kMassScale);
  if (target == 0ull) return clampk(1);
  const unsigned long long fm = sh.forced_mass;
  if (fm >= target) return clampk(npos);
  unsigned long long rem = target - fm;
  int above = npos;
  if (nfin == 0) return clampk(Np);
  if (stt.kmax == stt.kmin) {                               // all finite keys equal
    const unsigned long long m = mass_fixed(key_to_score(stt.kmax));
    if (m == 0ull || m * (unsigned long long)nfin < rem) return clampk(Np);
    return clampk(above + (int)((rem + m - 1) / m));
  }
  const uint32_t diff = stt.kmax ^ stt.kmin;
  const int hb = 31 - __clz((int)diff);
  uint32_t pmask = hb >= 31 ? 0u : ~((2u << hb) - 1u);
  uint32_t prefix = stt.kmax & pmask;
  int top = hb;
  int buf = 0;
  for (;;) {
    const int width = top + 1 < 8 ? top + 1 : 8;
    const int shift = top + 1 - width;
    const uint32_t dmask = (1u << width) - 1u;
    for_own_keys<NT>(keys, Np, [&](uint32_t key) {
      if ((key & pmask) == prefix && finite_key(key)) {
        const int bin = (key >> shift) & dmask;
        atomicAdd(&sh.hist[buf][bin], 1);
        atomicAdd(&sh.hmass[buf][bin], mass_fixed(key_to_score(key)));
      }
    });
    const int nb = buf == 2 ? 0 : buf + 1;
    if (tid < 256) { sh.hist[nb][tid] = 0; sh.hmass[nb][tid] = 0ull; }
    __syncthreads();
    // every wave scans the masses (digits descending) and finds the crossing bin
    int c[4], ctot = 0;
    unsigned long long mb[4], mtot = 0ull;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      c[i] = sh.hist[buf][255 - 4 * lane - i];
      mb[i] = sh.hmass[buf][255 - 4 * lane - i];
      ctot += c[i];
      mtot += mb[i];
    }
    unsigned long long minc = mtot;
#pragma unroll
    for (int off = 1; off < 64; off <<= 1) {
      const unsigned long long y = __shfl_up(minc, off);
      if (lane >= off) minc += y;
    }
    const int cinc = wave_incl_sum(ctot);
    const unsigned long long hit = __ballot(minc >= rem);
    if (hit == 0ull) return clampk(Np);                    // the finite keys never reach it
    const int first = __ffsll((long long)hit) - 1;
    unsigned long long mcum = minc - mtot;
    int ccum = cinc - ctot, dsel = 252 - 4 * lane, dcnt = c[3];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (mcum + mb[i] >= rem) { dsel = 255 - 4 * lane - i; dcnt = c[i]; break; }
      mcum += mb[i];
      ccum += c[i];
    }
    dsel = __builtin_amdgcn_readlane(dsel, first);
    dcnt = __builtin_amdgcn_readlane(dcnt, first);
    ccum = __builtin_amdgcn_readlane(ccum, first);
    const unsigned long long mc_lo = (unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)mcum, first);
    const unsigned long long mc_hi = (unsigned long long)(uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(mcum >> 32), first);
    mcum = mc_lo | (mc_hi << 32);
    prefix |= (uint32_t)dsel << shift;
    pmask |= dmask << shift;
    rem -= mcum;
    above += ccum;
    buf = nb;
    top -= width;
    if (top < 0) {
      // the crossing key: dcnt keys equal to `prefix`, each of mass m
      const unsigned long long m = mass_fixed(key_to_score(prefix));
      int need = m ? (int)((rem + m - 1) / m) : dcnt;
      need = need < dcnt ? need : dcnt;
      return clampk(above + need);
    }
  }
}

// Calls emit(p, pos) for every kept page p of [0, Np), pos = its rank in
// ascending page order.  Each thread walks a contiguous run of pages.
// Uses sh.wave_tot (and with WIDE sh.wpos) once (no barrier after it).  The
// two counts share one scan for Np < 2^15; WIDE scans them apart, for any Np.
template <int NT, bool WIDE = false, typename Emit>
__device__ __forceinline__ void select_compact(SelectLds<NT>& sh, const uint32_t* keys, int Np, uint32_t T,
                                               int take, Emit&& emit) {
  constexpr int NW = NT / 64;
  const int tid = threadIdx.x, lane = tid & 63;
  const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int chunk = (Np + NT - 1) / NT;
  const int lo = tid * chunk;
  const int hi = lo + chunk < Np ? lo + chunk : Np;
  int n_gt = 0, n_eq = 0;
  for (int p0 = lo; p0 < hi; p0 += 4) {
    uint32_t kv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kv[i] = p0 + i < hi ? keys[p0 + i] : 0u;   // 0: below every key
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      n_gt += kv[i] > T;
      n_eq += kv[i] == T;
    }
  }
  int gt_before, eq_before;
  if constexpr (!WIDE) {
    // one scan of both counts (each total is at most Np < 2^15)
    const int v = (n_gt << 16) | n_eq;
    const int incl = wave_incl_sum(v);
    if (lane == 63) sh.wave_tot[wave] = incl;
    __syncthreads();
    int before = incl - v;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) before += sh.wave_tot[w];
    gt_before = before >> 16;
    eq_before = before & 0xFFFF;
  } else {
    const int ig = wave_incl_sum(n_gt), ie = wave_incl_sum(n_eq);
    if (lane == 63) {
      sh.wave_tot[wave] = ig;
      sh.wpos[wave] = ie;
    }
    __syncthreads();
    gt_before = ig - n_gt;
    eq_before = ie - n_eq;
#pragma unroll
    for (int w = 0; w < NW; ++w)
      if (w < wave) {
        gt_before += sh.wave_tot[w];
        eq_before += sh.wpos[w];
      }
  }
  int take_eq = take - eq_before;
  take_eq = take_eq < 0 ? 0 : (take_eq > n_eq ? n_eq : take_eq);
  int pos = gt_before + (eq_before < take ? eq_before : take);
  int taken = 0;
  for (int p0 = lo; p0 < hi; p0 += 4) {
    uint32_t kv[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) kv[i] = p0 + i < hi ? keys[p0 + i] : 0u;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      if (kv[i] > T || (kv[i] == T && taken < take_eq)) {
        emit(p0 + i, pos++);
        taken += kv[i] == T;
      }
    }
  }
}

}  // namespace kvs
