// Device-side helpers shared by the gfx950 kernels: 16-bit conversions,
// MFMA operand types, wave-level reductions.  Internal to the library.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace kvs {

typedef __attribute__((__vector_size__(8 * sizeof(__bf16)))) __bf16 bf16x8_t;
typedef __attribute__((__vector_size__(8 * sizeof(_Float16)))) _Float16 f16x8_t;
typedef __attribute__((__vector_size__(4 * sizeof(float)))) float f32x4_t;
typedef __attribute__((__vector_size__(4 * sizeof(uint32_t)))) uint32_t u32x4_t;
typedef __attribute__((__vector_size__(2 * sizeof(uint32_t)))) uint32_t u32x2_t;

constexpr float kLog2e = 1.4426950408889634f;
constexpr float kLn2 = 0.6931471805599453f;

__device__ __forceinline__ float bf16_bits_to_f32(uint32_t b) { return __uint_as_float(b << 16); }

__device__ __forceinline__ float f16_bits_to_f32(uint32_t b) {
  return (float)__builtin_bit_cast(_Float16, (uint16_t)b);
}

template <bool F16>
__device__ __forceinline__ float h16_to_f32(uint32_t b) {
  if constexpr (F16) return f16_bits_to_f32(b);
  else return bf16_bits_to_f32(b);
}

// float32 -> bfloat16 bits, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}

// Low / high 16-bit halves of a packed pair as float32.
template <bool F16>
__device__ __forceinline__ float lo16(uint32_t w) { return h16_to_f32<F16>(w & 0xFFFFu); }
template <bool F16>
__device__ __forceinline__ float hi16(uint32_t w) {
  if constexpr (F16) return f16_bits_to_f32(w >> 16);
  else return __uint_as_float(w & 0xFFFF0000u);
}

__device__ __forceinline__ u32x4_t ld16(const void* p) { return *reinterpret_cast<const u32x4_t*>(p); }

// One 16x16x32 MFMA step.  A and B carry 8 16-bit values per lane; the k index
// of (lane, register) is the same for A and B, so any consistent assignment of
// head-dim elements to (lane group, register) computes the same contraction.
template <bool F16>
__device__ __forceinline__ f32x4_t mfma16(u32x4_t a, u32x4_t b, f32x4_t c) {
  if constexpr (F16)
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(f16x8_t, a),
                                                  __builtin_bit_cast(f16x8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                   __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

// Wave-local ordering of LDS writes before reads by other lanes of the same wave.
__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float readlane_f(float v, int lane) {
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), lane));
}

// Cross-lane steps through DPP (row_shr within 16-lane rows, row_bcast:15/31
// across rows) instead of LDS permutes.  Lanes whose source lies outside the
// pattern take `old`, the identity of the operation.  Every lane of the wave
// must be active.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp(int old, int x) {
  return __builtin_amdgcn_update_dpp(old, x, CTRL, ROWS, 0xF, false);
}

// Inclusive prefix sum in lane order.
__device__ __forceinline__ int wave_incl_sum(int x) {
  x += dpp<0x111, 0xF>(0, x);   // row_shr:1
  x += dpp<0x112, 0xF>(0, x);   // row_shr:2
  x += dpp<0x114, 0xF>(0, x);   // row_shr:4
  x += dpp<0x118, 0xF>(0, x);   // row_shr:8
  x += dpp<0x142, 0xA>(0, x);   // row_bcast:15 into rows 1 and 3
  x += dpp<0x143, 0xC>(0, x);   // row_bcast:31 into rows 2 and 3
  return x;
}

// Wave-wide reductions; the result is wave-uniform.
template <typename Op>
__device__ __forceinline__ int wave_reduce_i32(int x, int identity, Op op) {
  x = op(x, dpp<0x111, 0xF>(identity, x));
  x = op(x, dpp<0x112, 0xF>(identity, x));
  x = op(x, dpp<0x114, 0xF>(identity, x));
  x = op(x, dpp<0x118, 0xF>(identity, x));
  x = op(x, dpp<0x142, 0xA>(identity, x));
  x = op(x, dpp<0x143, 0xC>(identity, x));
  return __builtin_amdgcn_readlane(x, 63);
}

__device__ __forceinline__ int wave_sum_i32(int x) {
  return wave_reduce_i32(x, 0, [](int a, int b) { return a + b; });
}
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t x) {
  return (uint32_t)wave_reduce_i32((int)x, 0, [](int a, int b) { return (uint32_t)a > (uint32_t)b ? a : b; });
}
__device__ __forceinline__ uint32_t wave_min_u32(uint32_t x) {
  return (uint32_t)wave_reduce_i32((int)x, -1, [](int a, int b) { return (uint32_t)a < (uint32_t)b ? a : b; });
}
// fmaxf semantics: a NaN lane is dropped unless every lane is NaN.
__device__ __forceinline__ float wave_max_f32(float x) {
  return __int_as_float(wave_reduce_i32(__float_as_int(x), (int)0xFF800000u, [](int a, int b) {
    return __float_as_int(fmaxf(__int_as_float(a), __int_as_float(b)));
  }));
}
__device__ __forceinline__ float wave_sum_f32(float x) {
  return __int_as_float(wave_reduce_i32(__float_as_int(x), 0, [](int a, int b) {
    return __float_as_int(__int_as_float(a) + __int_as_float(b));
  }));
}

// max that propagates NaN from either side (fmaxf drops it).
__device__ __forceinline__ float nan_max(float a, float b) {
  return (a != a || a > b) ? a : b;
}

// (max, sum exp(x - max)) pairs: merge in a fixed order.
__device__ __forceinline__ void lse_merge(float& m, float& s, float m2, float s2) {
  const float M = fmaxf(m, m2);
  if (M == -INFINITY) { m = -INFINITY; s = 0.f; return; }
  s = s * __expf(m - M) + s2 * __expf(m2 - M);
  m = M;
}

}  // namespace kvs
