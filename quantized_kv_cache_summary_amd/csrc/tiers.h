// Decoding of packed page tiers, shared by the attention kernel, the
// standalone decode and the tier demotion.  ARGUS (argus_cache 0.1.7.1
// project page), "Why It Works: Storage vs. Computation": packed pages are
// rebuilt in registers just before use.  Codes are packed LSB first in
// head-dim order; every 32-element group of a token vector has a float16
// (scale, zero) pair.
#pragma once

#include "device.h"

namespace kvs {

// Loads `EL` consecutive codes of `BITS` bits starting at element e0 of a code row.
template <int EL, int BITS>
__device__ __forceinline__ void load_code_words(const uint8_t* rowp, int e0, uint32_t* w, int& shift0) {
  constexpr int NB = EL * BITS;   // bits to load
  const int bitoff = e0 * BITS;
  const uint8_t* p = rowp + (bitoff >> 3);
  shift0 = bitoff & 7;
  if constexpr (NB >= 32) {
#pragma unroll
    for (int i = 0; i < NB / 32; ++i) w[i] = reinterpret_cast<const uint32_t*>(p)[i];
  } else if constexpr (NB == 16) {
    w[0] = *reinterpret_cast<const uint16_t*>(p);
  } else {
    w[0] = *p;
  }
}

template <int BITS>
__device__ __forceinline__ uint32_t code_at(const uint32_t* w, int shift0, int e) {
  const int bit = shift0 + e * BITS;
  return (w[bit >> 5] >> (bit & 31)) & ((1u << BITS) - 1u);
}

// Decodes EL elements starting at e0 of token row `tokrow` of a packed page.
template <int D, int EL, int BITS>
__device__ __forceinline__ void decode_run(const uint8_t* codes, const uint16_t* sz, size_t tokrow,
                                           int e0, float* x) {
  uint32_t w[(EL * BITS + 31) / 32];
  int sh;
  load_code_words<EL, BITS>(codes + tokrow * (D * BITS / 8), e0, w, sh);
  const uint32_t szw = *reinterpret_cast<const uint32_t*>(sz + (tokrow * (D / 32) + e0 / 32) * 2);
  const float s = f16_bits_to_f32(szw & 0xFFFFu), z = f16_bits_to_f32(szw >> 16);
  if constexpr (BITS == 1) {
    const float zp = z + s, zm = z - s;
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] = code_at<1>(w, sh, e) ? zp : zm;
  } else {
#pragma unroll
    for (int e = 0; e < EL; ++e) x[e] = __builtin_fmaf((float)code_at<BITS>(w, sh, e), s, z);
  }
}

// Decodes EL FP8 (E4M3) codes, one byte each, starting at e0 of token row
// `tokrow`: x = e4m3(c) * s + z, exact (a 4-bit by 11-bit significand product)
// before the float32 rounding; the hardware's E4M3 conversion gives e4m3(c).
template <int D, int EL>
__device__ __forceinline__ void decode_fp8(const uint8_t* codes, const uint16_t* sz, size_t tokrow, int e0,
                                           float* x) {
  static_assert(EL == 4 || EL == 8, "runs of 4 or 8 codes");
  uint32_t w[EL / 4];
  const uint8_t* p = codes + tokrow * D + e0;
  if constexpr (EL == 8) {
    const u32x2_t t = *reinterpret_cast<const u32x2_t*>(p);
    w[0] = t[0];
    w[1] = t[1];
  } else {
    w[0] = *reinterpret_cast<const uint32_t*>(p);
  }
  const uint32_t szw = *reinterpret_cast<const uint32_t*>(sz + (tokrow * (D / 32) + e0 / 32) * 2);
  const float s = f16_bits_to_f32(szw & 0xFFFFu), z = f16_bits_to_f32(szw >> 16);
#pragma unroll
  for (int i = 0; i < EL / 4; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], false);
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8((int)w[i], true);
    x[4 * i + 0] = __builtin_fmaf(lo[0], s, z);
    x[4 * i + 1] = __builtin_fmaf(lo[1], s, z);
    x[4 * i + 2] = __builtin_fmaf(hi[0], s, z);
    x[4 * i + 3] = __builtin_fmaf(hi[1], s, z);
  }
}

// The 1-bit tier's outlier side table: replaces, in a decoded run
// [e0, e0 + EL) of one 32-element group, the element the group's word keeps
// (index in bits 0..4, float16 value in bits 16..31).
template <int EL>
__device__ __forceinline__ void apply_outlier(float* x, int e0, uint32_t word) {
  const int idx = (int)(word & 31u) - (e0 & 31);
  const float v = f16_bits_to_f32(word >> 16);
#pragma unroll
  for (int e = 0; e < EL; ++e) x[e] = e == idx ? v : x[e];
}

}  // namespace kvs
