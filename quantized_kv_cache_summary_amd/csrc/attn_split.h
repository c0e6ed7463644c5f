// Sparse paged decode attention over selected pages: the per-(row, split)
// body of the attention kernels (sparse_attn.hip), with the types and page
// decoding they share.  AMASS (amass-kv 0.1.1 project page),
// "AMASS": each decode step attends only to the pages that carry attention
// mass.  Packed tiers are rebuilt in registers just before use (ARGUS,
// argus_cache 0.1.7.1 project page, "Why It Works: Storage vs.
// Computation").  The design is described at the top of sparse_attn.hip.
#pragma once

#include <type_traits>

#include "device.h"
#include "launch.h"
#include "tiers.h"

namespace kvs {

// Waves per block: four (one per SIMD), which also read the pages.  The fused
// selector kernel has eight for up to four query heads per KV head (more would
// spill registers at two waves per SIMD), so that the latency-bound selection
// runs with two waves per SIMD; only the first four then read pages (a second
// wave per SIMD finishes its pages well after the first and the block's merge
// would wait for it).
template <int GM, bool SEL>
constexpr int attn_waves() { return SEL && GM <= 4 ? 8 : 4; }
constexpr int kStreamWaves = 4;

// Waves per SIMD a block must leave room for: the packed-tier kernel runs two
// 4-wave blocks per CU (its decode work hides the other block's latency), so
// its registers must fit two waves per SIMD.
template <int GM, bool TIERED, bool SEL>
constexpr int attn_min_waves_per_simd() { return (TIERED && !SEL && GM <= 4) ? 2 : 1; }

// The attention's LDS: per-wave probability tiles and the wave merge.
template <int W, int GM, int D>
struct AttnLds {
  float ptile[W][16][16];   // [wave][token][head]
  float wm[W][16], wl[W][16];
  float wacc[W][GM][D];
};

// Fused kernel's dynamic LDS, in 32-bit words: the split's share of the
// selection, then (16-byte aligned) the selector's state and the row's keys,
// whose space the attention's LDS reuses once the selection is done.
__host__ __device__ inline int sel_slice_words(int k_max, int n_splits) {
  return ((k_max + n_splits - 1) / n_splits + 1 + 3) & ~3;
}
constexpr int kBatch = 2;   // 16-token chunks per load batch; two batches are in flight

struct PagesDev {
  const uint16_t* k16;
  const uint16_t* v16;
  const uint8_t* kq[KV_NUM_PACKED_TIERS];
  const uint8_t* vq[KV_NUM_PACKED_TIERS];
  const uint16_t* ksz[KV_NUM_PACKED_TIERS];
  const uint16_t* vsz[KV_NUM_PACKED_TIERS];
  const uint32_t* page_entry;
  const uint16_t* v_hot;
  const int32_t* v_hot_slot;
  const uint16_t* k_hot;
  const uint32_t* kout;
  const uint32_t* vout;
};

// Device view of the caller's page pools.
inline PagesDev to_dev(const kv_pages& pg) {
  PagesDev d;
  d.k16 = (const uint16_t*)pg.k16;
  d.v16 = (const uint16_t*)pg.v16;
  for (int t = 0; t < KV_NUM_PACKED_TIERS; ++t) {
    d.kq[t] = pg.kq[t];
    d.vq[t] = pg.vq[t];
    d.ksz[t] = (const uint16_t*)pg.ksz[t];
    d.vsz[t] = (const uint16_t*)pg.vsz[t];
  }
  d.page_entry = pg.page_entry;
  d.v_hot = (const uint16_t*)pg.v_hot;
  d.v_hot_slot = pg.v_hot_slot;
  d.k_hot = (const uint16_t*)pg.k_hot;
  d.kout = pg.kout;
  d.vout = pg.vout;
  return d;
}

// Selector inputs and outputs of the fused kernel (unused without SEL).
struct SelArgs {
  const float* head_scores;   // [rows][G][max_pages]
  const float* lse_partial;   // [rows][n_tiles][G][2]
  float keep;
  int k_fixed;
  float coverage;             // < 0: budget mode (keep / k_fixed)
  int n_force_first, n_force_last, n_tiles;
  int32_t* sel;               // [rows][k_max], written by split 0
  int32_t* sel_count;         // [rows], written by split 0
  float* page_S;              // optional [rows][max_pages], written by split 0
};

template <int T>
struct TierTag {
  static constexpr int value = T;
};

template <int T>
constexpr int tier_bits() {
  return T == KV_TIER_I4 ? 4 : T == KV_TIER_I2 ? 2 : T == KV_TIER_B1 ? 1 : 8;
}

// Raw code words of one 16-token chunk of a page in packed tier T as the
// attention lanes read it: per MFMA k-step the codes of the lane's 8 key
// elements (key row `col`) and the (scale, zero) word of that row's group;
// per value slot j the codes of the lane's D/16 value elements and their
// (scale, zero) word.
template <int D, int T>
struct TierChunk {
  static constexpr int BITS = tier_bits<T>();
  static constexpr int KW = (8 * BITS + 31) / 32;
  static constexpr int VW = ((D / 16) * BITS + 31) / 32;
  uint32_t k[D / 32][KW];
  uint32_t ksz[D / 32];
  uint32_t v[4][VW];
  uint32_t vsz[4];
  uint32_t ko[D / 32];   // 1-bit outlier words, when the pools have side tables
  uint32_t vo[4];
};

// Exact 16-bit MFMA operand of two small values (codes, or E4M3 values): both
// have at most 8 significant bits, so bfloat16 truncation and float16
// conversion keep them exactly.
template <bool F16>
__device__ __forceinline__ uint32_t pack_exact(float lo, float hi) {
  if constexpr (F16) return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(lo, hi));
  else return __builtin_amdgcn_perm(__float_as_uint(hi), __float_as_uint(lo), 0x07060302u);
}

// byte i of w as float32 (one conversion instruction)
template <int I>
__device__ __forceinline__ float ubyte(uint32_t w) { return (float)((w >> (8 * I)) & 0xFFu); }

// The lane's 8 key codes of one k-step (elements 8 grp .. 8 grp + 7 of a
// 32-element group; their first bit is byte aligned) as the MFMA A operand:
// the codes themselves for the integer tiers (0 .. 2^b - 1) and the 1-bit
// tier (0, 1), the E4M3 values for FP8.  The group's scale and zero are
// applied to the MFMA result instead (tier_logits).
template <int T, bool F16>
__device__ __forceinline__ u32x4_t key_codes(const uint32_t* w) {
  u32x4_t a;
  if constexpr (T == KV_TIER_FP8) {
#pragma unroll
    for (int i = 0; i < 2; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
      a[2 * i] = pack_exact<F16>(lo[0], lo[1]);
      a[2 * i + 1] = pack_exact<F16>(hi[0], hi[1]);
    }
  } else if constexpr (T == KV_TIER_I8) {
    a[0] = pack_exact<F16>(ubyte<0>(w[0]), ubyte<1>(w[0]));
    a[1] = pack_exact<F16>(ubyte<2>(w[0]), ubyte<3>(w[0]));
    a[2] = pack_exact<F16>(ubyte<0>(w[1]), ubyte<1>(w[1]));
    a[3] = pack_exact<F16>(ubyte<2>(w[1]), ubyte<3>(w[1]));
  } else if constexpr (T == KV_TIER_I4) {
    const uint32_t lo = w[0] & 0x0F0F0F0Fu, hi = (w[0] >> 4) & 0x0F0F0F0Fu;   // elements 2i, 2i + 1
    a[0] = pack_exact<F16>(ubyte<0>(lo), ubyte<0>(hi));
    a[1] = pack_exact<F16>(ubyte<1>(lo), ubyte<1>(hi));
    a[2] = pack_exact<F16>(ubyte<2>(lo), ubyte<2>(hi));
    a[3] = pack_exact<F16>(ubyte<3>(lo), ubyte<3>(hi));
  } else if constexpr (T == KV_TIER_I2) {
    float f[8];
#pragma unroll
    for (int k = 0; k < 4; ++k) {                  // byte 0: element k, byte 1: element 4 + k
      const uint32_t m = (w[0] >> (2 * k)) & 0x0303u;
      f[k] = ubyte<0>(m);
      f[4 + k] = ubyte<1>(m);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = pack_exact<F16>(f[2 * i], f[2 * i + 1]);
  } else {                                         // 1-bit: 1.0 where the bit is set
    constexpr uint32_t one = F16 ? 0x3C00u : 0x3F80u;
#pragma unroll
    for (int i = 0; i < 4; ++i)
      a[i] = (((w[0] >> (2 * i)) & 1u) | (((w[0] >> (2 * i + 1)) & 1u) << 16)) * one;
  }
  return a;
}

// Scale and zero of a packed group's codes from its (scale, zero) float16
// word: x = sc * c + ze, so (s, z) for the integer tiers and FP8 and (2 s,
// z - s) for the 1-bit tier (x = z - s + 2 s c).
template <int T>
__device__ __forceinline__ void group_scale_zero(uint32_t szw, float& sc, float& ze) {
  const float s = f16_bits_to_f32(szw & 0xFFFFu), z = f16_bits_to_f32(szw >> 16);
  if constexpr (T == KV_TIER_B1) {
    sc = 2.f * s;
    ze = z - s;
  } else {
    sc = s;
    ze = z;
  }
}

// 1-bit outlier side table on the key side: the kept element (index in bits
// 0..4 of `word`, float16 value in bits 16..31) of the group, if it is one of
// the lane's 8 elements (8 grp .. 8 grp + 7), is given in code units of the
// group, c' = (v - (z - s)) / (2 s), as a 16-bit hi part (replacing its code
// in `a`) and a 16-bit lo remainder (`lo`, zero elsewhere), so the group's
// scale and zero turn the MFMA result into the kept value.  A group with
// s = 0 keeps its code: then every element is within 2^-20 of z, the kept
// value too.
template <bool F16>
__device__ __forceinline__ void outlier_operand(u32x4_t& a, u32x4_t& lo, uint32_t word, uint32_t szw, int grp) {
  const int idx = (int)(word & 31u) - 8 * grp;
  float sc, ze;
  group_scale_zero<KV_TIER_B1>(szw, sc, ze);
  const float v = f16_bits_to_f32(word >> 16);
  const bool mine = idx >= 0 && idx < 8 && sc != 0.f;
  const float c = mine ? (v - ze) * __builtin_amdgcn_rcpf(sc) : 0.f;
  uint32_t h16, l16;
  if constexpr (F16) {
    const _Float16 h = (_Float16)c;
    h16 = __builtin_bit_cast(uint16_t, h);
    l16 = __builtin_bit_cast(uint16_t, (_Float16)(c - (float)h));
  } else {
    h16 = f32_to_bf16_rne(c);
    l16 = f32_to_bf16_rne(c - __uint_as_float(h16 << 16));
  }
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    const uint32_t m = !mine ? 0u : (idx == 2 * w ? 0x0000FFFFu : (idx == 2 * w + 1 ? 0xFFFF0000u : 0u));
    const uint32_t hv = h16 | (h16 << 16), lv = l16 | (l16 << 16);
    a[w] = (a[w] & ~m) | (hv & m);
    lo[w] = lv & m;
  }
}

// Requests the codes of EL elements from e0 of token row `tokrow` of packed
// tier T and the group's (scale, zero) word.
template <int D, int EL, int T>
__device__ __forceinline__ void tier_load(const uint8_t* codes, const uint16_t* sz, size_t tokrow, int e0,
                                          uint32_t* w, uint32_t& szw) {
  constexpr int BITS = tier_bits<T>();
  szw = *reinterpret_cast<const uint32_t*>(sz + (tokrow * (D / 32) + e0 / 32) * 2);
  int sh;
  load_code_words<EL, BITS>(codes + tokrow * (D * BITS / 8), e0, w, sh);
}

// Decodes what tier_load requested: int-b x = c*s + z (one FMA), 1-bit
// x = z +- s, FP8 x = e4m3(c)*s + z.  Codes are taken out of their words a
// byte at a time where the run's first bit is byte aligned.
template <int EL, int T>
__device__ __forceinline__ void tier_decode(const uint32_t* w, uint32_t szw, int e0, float* x) {
  constexpr int BITS = tier_bits<T>();
  const float s = f16_bits_to_f32(szw & 0xFFFFu), z = f16_bits_to_f32(szw >> 16);
  constexpr bool aligned = (EL * BITS) % 8 == 0;   // runs start at multiples of EL
  const int sh = aligned ? 0 : (e0 * BITS) & 7;
  if constexpr (T == KV_TIER_I8 && EL % 4 == 0) {
#pragma unroll
    for (int i = 0; i < EL / 4; ++i) {
      x[4 * i + 0] = __builtin_fmaf(ubyte<0>(w[i]), s, z);
      x[4 * i + 1] = __builtin_fmaf(ubyte<1>(w[i]), s, z);
      x[4 * i + 2] = __builtin_fmaf(ubyte<2>(w[i]), s, z);
      x[4 * i + 3] = __builtin_fmaf(ubyte<3>(w[i]), s, z);
    }
  } else if constexpr (T == KV_TIER_I4 && EL == 8) {
    const uint32_t lo = w[0] & 0x0F0F0F0Fu, hi = (w[0] >> 4) & 0x0F0F0F0Fu;
    x[0] = __builtin_fmaf(ubyte<0>(lo), s, z);
    x[1] = __builtin_fmaf(ubyte<0>(hi), s, z);
    x[2] = __builtin_fmaf(ubyte<1>(lo), s, z);
    x[3] = __builtin_fmaf(ubyte<1>(hi), s, z);
    x[4] = __builtin_fmaf(ubyte<2>(lo), s, z);
    x[5] = __builtin_fmaf(ubyte<2>(hi), s, z);
    x[6] = __builtin_fmaf(ubyte<3>(lo), s, z);
    x[7] = __builtin_fmaf(ubyte<3>(hi), s, z);
  } else if constexpr (T == KV_TIER_I2 && EL == 8) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
      const uint32_t m = (w[0] >> (2 * k)) & 0x0303u;
      x[k] = __builtin_fmaf(ubyte<0>(m), s, z);
      x[4 + k] = __builtin_fmaf(ubyte<1>(m), s, z);
    }
  } else if constexpr (T == KV_TIER_FP8) {
#pragma unroll
    for (int i = 0; i < EL / 4; ++i) {
      const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
      const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
      x[4 * i + 0] = __builtin_fmaf(lo[0], s, z);
      x[4 * i + 1] = __builtin_fmaf(lo[1], s, z);
      x[4 * i + 2] = __builtin_fmaf(hi[0], s, z);
      x[4 * i + 3] = __builtin_fmaf(hi[1], s, z);
    }
  } else if constexpr (T == KV_TIER_B1) {
    const float zp = z + s, zm = z - s;
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] = code_at<1>(w, sh, e) ? zp : zm;
  } else {
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] = __builtin_fmaf((float)code_at<BITS>(w, sh, e), s, z);
  }
}

// ---------------------------------------------------------------- the kernel

// Per-wave attention state: running max (per head, shared by the four lane
// groups), this lane's partial softmax sum, and acc[head][d/16] of the
// token slot / element chunk this lane owns.
template <int D, int GM>
struct AttnState {
  static constexpr int EV = D / 16;
  float m_run;
  float l_run;
  float acc[GM][EV];
};

// Softmax update for one 16-token chunk given its raw logits (head col,
// tokens 4*grp + i); writes the probabilities to the wave's LDS tile.
template <int D, int GM>
__device__ __forceinline__ void softmax_chunk(AttnState<D, GM>& st, const f32x4_t& zacc, int tok0, int L,
                                              bool page_ok, float scale_log2, float (*ptile)[16],
                                              int grp, int col) {
  constexpr int EV = D / 16;
  constexpr float kRescale = 8.0f;
  float z[4];
  float cm = -INFINITY;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tpos = tok0 + 4 * grp + i;
    z[i] = (page_ok && tpos < L) ? zacc[i] * scale_log2 : -INFINITY;
    cm = nan_max(cm, z[i]);
  }
  cm = nan_max(cm, __shfl_xor(cm, 16));
  cm = nan_max(cm, __shfl_xor(cm, 32));
  // a NaN logit (NaN query) makes the running max NaN, so the head's output
  // and lse come out NaN instead of being dropped
  const float m_new = nan_max(st.m_run, cm);
  const bool need = (m_new > st.m_run + kRescale) || (m_new != m_new && st.m_run == st.m_run);
  if (__ballot(need)) {
    const float alpha = (m_new == -INFINITY) ? 1.f : __builtin_amdgcn_exp2f(st.m_run - m_new);
    if (m_new != -INFINITY) st.m_run = m_new;
    st.l_run *= alpha;
#pragma unroll
    for (int h = 0; h < GM; ++h) {
      const float ah = readlane_f(alpha, h);
#pragma unroll
      for (int e = 0; e < EV; ++e) st.acc[h][e] *= ah;
    }
  }
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const float pz = (st.m_run == -INFINITY) ? 0.f : __builtin_amdgcn_exp2f(z[i] - st.m_run);
    st.l_run += pz;
    ptile[4 * grp + i][col] = pz;
  }
  wave_lds_sync();
}

// acc[h][:] += p[h][token] * v for one token slot of the chunk.
template <int D, int GM>
__device__ __forceinline__ void pv_accumulate(AttnState<D, GM>& st, const float* v, const float (*ptile)[16], int tk) {
  constexpr int EV = D / 16;
  float pv[GM];
#pragma unroll
  for (int h4 = 0; h4 < GM; h4 += 4) {
    const float4 t4 = *reinterpret_cast<const float4*>(&ptile[tk][h4]);
    pv[h4] = t4.x; pv[h4 + 1] = t4.y; pv[h4 + 2] = t4.z; pv[h4 + 3] = t4.w;
  }
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < EV; ++e) st.acc[h][e] = __builtin_fmaf(pv[h], v[e], st.acc[h][e]);
}

template <bool F16, int EV>
__device__ __forceinline__ void unpack_v(const u32x4_t& r, float* v) {
  if constexpr (EV == 8) {
#pragma unroll
    for (int w = 0; w < 4; ++w) { v[2 * w] = lo16<F16>(r[w]); v[2 * w + 1] = hi16<F16>(r[w]); }
  } else {
#pragma unroll
    for (int w = 0; w < 2; ++w) { v[2 * w] = lo16<F16>(r[w]); v[2 * w + 1] = hi16<F16>(r[w]); }
  }
}

// Raw loads of one 16-token chunk of a native page: K rows for the MFMA (key
// row `col`, 64 contiguous bytes per k-step), V rows for the PV lanes (token
// 4j + grp, 16 contiguous bytes per lane).
template <int D>
struct ChunkRaw {
  u32x4_t k[D / 32];
  u32x4_t v[4];
};

template <int D>
__device__ __forceinline__ void load_native_chunk(ChunkRaw<D>& r, const uint16_t* kbase, const uint16_t* vbase,
                                                  int c, int col, int grp) {
  constexpr int KS = D / 32, EV = D / 16;
  const uint16_t* kp = kbase + (size_t)(c * 16 + col) * D + 8 * grp;
#pragma unroll
  for (int s = 0; s < KS; ++s) r.k[s] = ld16(kp + 32 * s);
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const uint16_t* vp = vbase + (size_t)(c * 16 + 4 * j + grp) * D + col * EV;
    if constexpr (EV == 8) r.v[j] = ld16(vp);
    else {
      const u32x2_t t = *reinterpret_cast<const u32x2_t*>(vp);
      r.v[j] = u32x4_t{t[0], t[1], 0, 0};
    }
  }
}

// Attention of one (row, split): the split's share [beg, end) of the row's
// cnt selected pages (list: the share itself, in LDS, with LDS_LIST; else the
// row's whole selection in device memory), dealt round-robin to the first
// kStreamWaves waves of the block; then the wave merge, this split's partial,
// and the row's split merge by the last split to finish.  `clear` (may be
// NULL) is a per-row word the merging block resets with the split counter.
// Every thread of the block calls it; qop is the lane's query operand.
template <int D, int GM, bool F16, bool TIERED, bool LDS_LIST, int kThreads>
__device__ __forceinline__ void attend_split(const PagesDev& pg, const int32_t* __restrict__ block_table,
                                             int Hkv, int G, int P, int max_pages, int row, int split,
                                             int n_splits, int cnt,
                                             const int32_t* list, int L, int Np, const u32x4_t (&qop)[D / 32],
                                             float scale_log2, float* __restrict__ partials,
                                             unsigned* __restrict__ counters, unsigned* clear,
                                             float* __restrict__ out, float* __restrict__ lse,
                                             AttnLds<kStreamWaves, GM, D>* al) {
  constexpr int KS = D / 32;     // MFMA k-steps
  constexpr int EV = D / 16;     // value elements per lane
  const int b = row / Hkv, g = row - b * Hkv;
  const int lane = threadIdx.x & 63;
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);   // wave-uniform (SGPR)
  const int col = lane & 15, grp = lane >> 4;

  const int beg = (int)(((long long)split * cnt) / n_splits);
  const int end = (int)(((long long)(split + 1) * cnt) / n_splits);
  const int n_mine =
      wave < kStreamWaves && end - beg > wave ? (end - beg - wave + kStreamWaves - 1) / kStreamWaves : 0;

  AttnState<D, GM> st;
  st.m_run = -INFINITY;
  st.l_run = 0.f;
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < EV; ++e) st.acc[h][e] = 0.f;

  // tiered kernels: sum of each 32-element group of the lane's query head
  // (column col), for the zero terms of packed keys
  float qsum[KS];
#pragma unroll
  for (int s = 0; s < KS; ++s) {
    float t = 0.f;
    if constexpr (TIERED) {
#pragma unroll
      for (int w = 0; w < 4; ++w) t += lo16<F16>(qop[s][w]) + hi16<F16>(qop[s][w]);
      t += __shfl_xor(t, 16);
      t += __shfl_xor(t, 32);
    }
    qsum[s] = t;
  }

  const int32_t* bt = block_table + (size_t)b * max_pages;
  const size_t page_elems = (size_t)P * D;
  const int cpp = P / 16;   // 16-token chunks per page
  float (*pt)[16] = al->ptile[wave < kStreamWaves ? wave : 0];   // used by streaming waves only

  if constexpr (!TIERED) {
    for (int j0 = 0; j0 < n_mine; j0 += 64) {
      const int nb = n_mine - j0 < 64 ? n_mine - j0 : 64;
      // this wave's pages, one per lane: logical page, slot, hot-buffer slot
      int l_p = -1, l_hot = -1;
      uint32_t l_slot = 0;
      if (lane < nb) {
        const int li = wave + kStreamWaves * (j0 + lane);
        const int p = LDS_LIST ? list[li] : list[beg + li];
        if (p >= 0 && p < Np) {
          l_p = p;
          const int phys = bt[p];
          l_slot = (uint32_t)phys;
          if (pg.v_hot_slot) l_hot = pg.v_hot_slot[(size_t)phys * Hkv + g];
        }
      }
      const unsigned long long valid = __ballot(l_p >= 0);
      if (valid == 0) continue;

      // skipped entries read the first valid page of the list instead (and are
      // masked), so every load of a batch is unconditional straight-line code
      const int first = __ffsll((long long)valid) - 1;
      if (l_p < 0) {
        l_slot = (uint32_t)__builtin_amdgcn_readlane((int)l_slot, first);
        l_hot = __builtin_amdgcn_readlane(l_hot, first);
      }
      const int nch = nb * cpp;
      // issue the loads of chunks [cb, cb + NB) into r (the last chunk is
      // re-read past the end; those extra chunks are never computed)
      auto issue = [&](ChunkRaw<D> (&r)[kBatch], int (&pp)[kBatch], int cb) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          const int ci = cb + u < nch ? cb + u : nch - 1;
          const int jj = ci / cpp;
          pp[u] = __builtin_amdgcn_readlane(l_p, jj);
          const uint32_t slot = (uint32_t)__builtin_amdgcn_readlane((int)l_slot, jj);
          const int hot = __builtin_amdgcn_readlane(l_hot, jj);
          const size_t pr = (size_t)slot * Hkv + g;
          const size_t hr = (size_t)hot * page_elems;
          const uint16_t* kb = hot >= 0 && pg.k_hot ? pg.k_hot + hr : pg.k16 + pr * page_elems;
          const uint16_t* vb = hot >= 0 ? pg.v_hot + hr : pg.v16 + pr * page_elems;
          load_native_chunk<D>(r[u], kb, vb, ci - jj * cpp, col, grp);
        }
      };
      auto compute = [&](const ChunkRaw<D> (&r)[kBatch], const int (&pp)[kBatch], int cb) {
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
          if (cb + u >= nch) break;
          const int ci = cb + u;
          const int c = ci - (ci / cpp) * cpp;
          const int p = pp[u];
          f32x4_t zacc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int s = 0; s < KS; ++s) zacc = mfma16<F16>(r[u].k[s], qop[s], zacc);
          const int tok0 = p * P + c * 16;
          softmax_chunk<D, GM>(st, zacc, tok0, L, p >= 0, scale_log2, pt, grp, col);
          // values of tokens that do not exist (past seq_len, skipped entries)
          // are zeroed: their probability is 0 but the memory may hold NaN
          const bool full = p >= 0 && tok0 + 16 <= L;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            float v[EV];
            unpack_v<F16, EV>(r[u].v[j], v);
            if (!full) {
              const uint32_t vk = (p >= 0 && tok0 + 4 * j + grp < L) ? 0xFFFFFFFFu : 0u;
#pragma unroll
              for (int e = 0; e < EV; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) & vk);
            }
            pv_accumulate<D, GM>(st, v, pt, 4 * j + grp);
          }
          wave_lds_sync();
        }
      };
      ChunkRaw<D> ra[kBatch], rb[kBatch];
      int pa[kBatch], pb[kBatch];
      issue(ra, pa, 0);
      for (int cb = 0; cb < nch; cb += 2 * kBatch) {
        if (cb + kBatch < nch) issue(rb, pb, cb + kBatch);
        __builtin_amdgcn_sched_barrier(0);
        compute(ra, pa, cb);
        if (cb + kBatch < nch) {
          if (cb + 2 * kBatch < nch) issue(ra, pa, cb + 2 * kBatch);
          __builtin_amdgcn_sched_barrier(0);
          compute(rb, pb, cb + kBatch);
        }
      }
    }
  } else {
    // Tiered pages: the wave's pages in batches of 64 (one per lane), each
    // batch taken tier by tier so that every loop below has one load shape.
    for (int j0 = 0; j0 < n_mine; j0 += 64) {
      const int nb = n_mine - j0 < 64 ? n_mine - j0 : 64;
      int l_p = -1, l_hot = -1;
      uint32_t l_tier = 7, l_slot = 0;   // 7: not a valid entry
      if (lane < nb) {
        const int li = wave + kStreamWaves * (j0 + lane);
        const int p = LDS_LIST ? list[li] : list[beg + li];
        if (p >= 0 && p < Np) {
          l_p = p;
          const int phys = bt[p];
          l_slot = (uint32_t)phys;
          l_tier = KV_TIER_NATIVE;
          if (pg.page_entry) {
            const uint32_t e = pg.page_entry[phys];
            l_tier = e >> 29;
            l_slot = e & 0x1FFFFFFFu;
          }
          if (pg.v_hot_slot) l_hot = pg.v_hot_slot[(size_t)phys * Hkv + g];
        }
      }
      auto run_tier = [&](auto tc) {
        constexpr int T = decltype(tc)::value;
        using Raw = typename std::conditional<T == KV_TIER_NATIVE, ChunkRaw<D>, TierChunk<D, T>>::type;
        const unsigned long long mask = __ballot(l_p >= 0 && l_tier == (uint32_t)T);
        if (mask == 0) return;
        const int nu = __popcll(mask) * cpp;
        // units in list order; past the last one the iterator repeats it (a
        // request whose result is never computed), so every load below is
        // unconditional and the wait counts do not depend on the path
        unsigned long long it = mask;
        int it_c = 0, last_lane = __ffsll((long long)mask) - 1, last_c = 0;
        auto next = [&](int& lane_out, int& c_out) {
          if (it == 0) {
            lane_out = last_lane;
            c_out = last_c;
            return;
          }
          lane_out = last_lane = __ffsll((long long)it) - 1;
          c_out = last_c = it_c;
          if (++it_c == cpp) {
            it_c = 0;
            it &= it - 1;
          }
        };
        auto issue = [&](Raw& r, int jj, int c) {
          const uint32_t slot = (uint32_t)__builtin_amdgcn_readlane((int)l_slot, jj);
          const size_t pr = (size_t)slot * Hkv + g;
          if constexpr (T == KV_TIER_NATIVE) {
            const int hot = __builtin_amdgcn_readlane(l_hot, jj);
            const size_t hr = (size_t)hot * page_elems;
            const uint16_t* kbase = hot >= 0 && pg.k_hot ? pg.k_hot + hr : pg.k16 + pr * page_elems;
            const uint16_t* vbase = hot >= 0 ? pg.v_hot + hr : pg.v16 + pr * page_elems;
            load_native_chunk<D>(r, kbase, vbase, c, col, grp);
          } else {
            constexpr int BITS = tier_bits<T>();
            const size_t tok = pr * P + c * 16;
            const uint8_t* kc = pg.kq[T - 1] + (tok + col) * (D * BITS / 8);
            const uint16_t* ks = pg.ksz[T - 1];
#pragma unroll
            for (int s = 0; s < KS; ++s) {
              int sh;   // 0: the lane's 8 codes start on a byte boundary
              load_code_words<8, BITS>(kc, 32 * s + 8 * grp, r.k[s], sh);
            }
            {
              const uint32_t* w = reinterpret_cast<const uint32_t*>(ks + (tok + col) * (D / 32) * 2);
#pragma unroll
              for (int s = 0; s < KS; ++s) r.ksz[s] = w[s];
            }
#pragma unroll
            for (int j = 0; j < 4; ++j)
              tier_load<D, EV, T>(pg.vq[T - 1], pg.vsz[T - 1], tok + 4 * j + grp, col * EV, r.v[j], r.vsz[j]);
            if constexpr (T == KV_TIER_B1) {
              if (pg.kout) {
#pragma unroll
                for (int s = 0; s < KS; ++s) r.ko[s] = pg.kout[(tok + col) * (D / 32) + s];
#pragma unroll
                for (int j = 0; j < 4; ++j) r.vo[j] = pg.vout[(tok + 4 * j + grp) * (D / 32) + (col * EV) / 32];
              }
            }
          }
        };
        auto compute = [&](const Raw& r, int jj, int c) {
          const int p = __builtin_amdgcn_readlane(l_p, jj);
          const int tok0 = p * P + c * 16;
          f32x4_t zacc = {0.f, 0.f, 0.f, 0.f};
          if constexpr (T == KV_TIER_NATIVE) {
#pragma unroll
            for (int s = 0; s < KS; ++s) zacc = mfma16<F16>(r.k[s], qop[s], zacc);
          } else {
            // q.k of a packed key: per 32-element group, s q.c + z sum(q) (1-bit:
            // 2 s q.c + (z - s) sum(q)), the codes c exact in the 16-bit MFMA
            // operand, one MFMA per group, scale and zero applied to its result
            // the MFMA leaves token 4 grp + i in this lane: its (scale, zero)
            // word comes from lane 4 grp + i (key row 4 grp + i) by a permute
#pragma unroll
            for (int s = 0; s < KS; ++s) {
              u32x4_t a = key_codes<T, F16>(r.k[s]);
              const f32x4_t z0 = {0.f, 0.f, 0.f, 0.f};
              f32x4_t part;
              if constexpr (T == KV_TIER_B1) {
                if (pg.kout) {
                  u32x4_t alo;
                  outlier_operand<F16>(a, alo, r.ko[s], r.ksz[s], grp);
                  part = mfma16<F16>(alo, qop[s], mfma16<F16>(a, qop[s], z0));
                } else {
                  part = mfma16<F16>(a, qop[s], z0);
                }
              } else {
                part = mfma16<F16>(a, qop[s], z0);
              }
#pragma unroll
              for (int i = 0; i < 4; ++i) {
                const uint32_t w = (uint32_t)__builtin_amdgcn_ds_bpermute((4 * grp + i) * 4, (int)r.ksz[s]);
                float sc, ze;
                group_scale_zero<T>(w, sc, ze);
                zacc[i] = __builtin_fmaf(sc, part[i], __builtin_fmaf(ze, qsum[s], zacc[i]));
              }
            }
          }
          softmax_chunk<D, GM>(st, zacc, tok0, L, true, scale_log2, pt, grp, col);
          const bool full = tok0 + 16 <= L;
#pragma unroll
          for (int j = 0; j < 4; ++j) {
            const int tk = 4 * j + grp;
            float v[EV];
            if constexpr (T == KV_TIER_NATIVE) unpack_v<F16, EV>(r.v[j], v);
            else {
              tier_decode<EV, T>(r.v[j], r.vsz[j], col * EV, v);
              if constexpr (T == KV_TIER_B1)
                if (pg.vout) apply_outlier<EV>(v, col * EV, r.vo[j]);
            }
            // values of tokens past seq_len are zeroed: probability 0, memory may hold NaN
            if (!full) {
              const uint32_t vk = tok0 + tk < L ? 0xFFFFFFFFu : 0u;
#pragma unroll
              for (int e = 0; e < EV; ++e) v[e] = __uint_as_float(__float_as_uint(v[e]) & vk);
            }
            pv_accumulate<D, GM>(st, v, pt, tk);
          }
          wave_lds_sync();
        };
        Raw ra, rb;
        int ja, ca, jb, cb;
        next(ja, ca);
        issue(ra, ja, ca);
        int u = 0;
        for (; u + 2 <= nu; u += 2) {
          next(jb, cb);
          issue(rb, jb, cb);
          __builtin_amdgcn_sched_barrier(0);
          compute(ra, ja, ca);
          next(ja, ca);
          issue(ra, ja, ca);
          __builtin_amdgcn_sched_barrier(0);
          compute(rb, jb, cb);
        }
        if (u < nu) compute(ra, ja, ca);
      };
      run_tier(TierTag<KV_TIER_NATIVE>{});
      run_tier(TierTag<KV_TIER_FP8>{});
      run_tier(TierTag<KV_TIER_I8>{});
      run_tier(TierTag<KV_TIER_I4>{});
      run_tier(TierTag<KV_TIER_I2>{});
      run_tier(TierTag<KV_TIER_B1>{});
    }
  }

  // ---- wave totals: l over lane groups, acc over token slots
  float l_run = st.l_run;
  l_run += __shfl_xor(l_run, 16);
  l_run += __shfl_xor(l_run, 32);
#pragma unroll
  for (int h = 0; h < GM; ++h)
#pragma unroll
    for (int e = 0; e < EV; ++e) {
      float a = st.acc[h][e];
      a += __shfl_xor(a, 16);
      a += __shfl_xor(a, 32);
      st.acc[h][e] = a;
    }
  if (wave < kStreamWaves && lane < 16) { al->wm[wave][lane] = st.m_run; al->wl[wave][lane] = l_run; }
  if (wave < kStreamWaves && grp == 0) {
#pragma unroll
    for (int h = 0; h < GM; ++h)
#pragma unroll
      for (int e = 0; e < EV; ++e) al->wacc[wave][h][col * EV + e] = st.acc[h][e];
  }
  __syncthreads();

  // ---- merge the waves (fixed order) and write this split's partial
  float* dst = partials + ((size_t)row * n_splits + split) * G * (D + 2);
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, e = idx - h * D;
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < kStreamWaves; ++w) M = nan_max(M, al->wm[w][h]);
    float a = 0.f, l = 0.f;
    if (M != -INFINITY) {
#pragma unroll
      for (int w = 0; w < kStreamWaves; ++w) {
        const float f = exp2f(al->wm[w][h] - M);
        a += al->wacc[w][h][e] * f;
        l += al->wl[w][h] * f;
      }
    }
    // device-coherent stores (written through to the chip's coherence point),
    // so another block may read them after the counter below says so
    __hip_atomic_store(dst + (size_t)h * (D + 2) + e, a, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (e == 0) {
      __hip_atomic_store(dst + (size_t)h * (D + 2) + D, M, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      __hip_atomic_store(dst + (size_t)h * (D + 2) + D + 1, l, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }

  // ---- the last split of the row to finish merges all splits in split order.
  // Every partial store above has completed before the count is raised, and
  // the merging block reads partials with device-coherent loads; no cache
  // write-back fence is needed because nothing else crosses blocks.
  __shared__ int is_last;
  __builtin_amdgcn_s_waitcnt(0);
  __syncthreads();
  if (threadIdx.x == 0)
    is_last = __hip_atomic_fetch_add(&counters[row], 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
              (unsigned)(n_splits - 1);
  __syncthreads();
  if (!is_last) return;
  const float* src = partials + (size_t)row * n_splits * G * (D + 2);
  const size_t stride = (size_t)G * (D + 2);
  for (int idx = threadIdx.x; idx < G * D; idx += kThreads) {
    const int h = idx / D, e = idx - h * D;
    const float* sh = src + (size_t)h * (D + 2);
    constexpr int U = 8;
    float M = -INFINITY, a = 0.f, l = 0.f;
    for (int s0 = 0; s0 < n_splits; s0 += U) {
      float av[U], mv[U], lv[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int si = s0 + u < n_splits ? s0 + u : n_splits - 1;
        av[u] = __hip_atomic_load(sh + si * stride + e, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        mv[u] = __hip_atomic_load(sh + si * stride + D, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        lv[u] = __hip_atomic_load(sh + si * stride + D + 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (s0 + u >= n_splits) break;
        const float Mn = nan_max(M, mv[u]);
        if (Mn == -INFINITY) continue;
        const float fo = exp2f(M - Mn), fn = exp2f(mv[u] - Mn);
        a = a * fo + av[u] * fn;
        l = l * fo + lv[u] * fn;
        M = Mn;
      }
    }
    const size_t hq = (size_t)b * Hkv * G + (size_t)g * G + h;
    const bool empty = l == 0.f;
    out[hq * D + e] = empty ? 0.f : a / l;
    if (e == 0) lse[hq] = empty ? -INFINITY : (M + log2f(l)) * kLn2;
  }
  if (threadIdx.x == 0) {
    __hip_atomic_store(&counters[row], 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (clear) __hip_atomic_store(clear, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  }
}

}  // namespace kvs
