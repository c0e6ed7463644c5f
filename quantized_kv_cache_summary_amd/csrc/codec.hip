// Packed low-bit page tiers: encoder.  ARGUS (argus_cache 0.1.7.1 project
// page), "Visual Architecture" and the tier legend: INT8, INT4 (2-way
// bit-packed), INT2 (4-way bit-packed), 1-bit (8-way sign-packed).
//
// Per token vector, per group of 32 consecutive head-dim elements, with every
// operation an IEEE float32 operation rounded to nearest even and no fused
// multiply-add (this file is compiled with -ffp-contract=off; division and
// square root are the correctly rounded ones):
//   int-b: s = f16(f32(max - min) / (2^b - 1)), z = f16(min),
//          c = 0 if s == 0 else clamp(rint(f32(x - z) / s), 0, 2^b - 1)
//   1-bit: z = f16(T(x) / 32), s = f16(T(|x - z|) / 32), c = (x >= z)
//          with T the pairwise tree sum, level by level, pairs (2i, 2i+1)
//   f16(): round to nearest even, saturating at +-65504.
//   FP8 (the cascade's first step below 16 bits, "gentle precision" in the
//   tier legend; format read as OCP E4M3, finite variant): s = f16(max|x| /
//   448), z = 0, c = 0 if s == 0 else e4m3(f32(x / s)), one code per byte.
// Codes are packed LSB first in head-dim order; (s, z) are stored as a float16
// pair per group.  One thread encodes one group.

#include "device.h"
#include "launch.h"
#include "tiers.h"

namespace kvs {

__device__ __forceinline__ float f16_sat(float x) {
  x = fminf(fmaxf(x, -65504.f), 65504.f);
  return (float)(_Float16)x;
}

__device__ __forceinline__ uint16_t f16_bits(float x) {
  return __builtin_bit_cast(uint16_t, (_Float16)x);
}

// float32 -> E4M3 code: nearest finite value, ties to the even code, |y| >= 448
// saturating to 448 (0x7E), the sign bit copied from y.  Below 2^-6 the codes
// are the subnormal multiples of 2^-9 (|y| * 512 is exact, then rounded to an
// integer half to even); above, the float32 pattern is rounded half to even at
// the 3rd mantissa bit and the exponent rebiased from 127 to 7.
__device__ __forceinline__ uint32_t f32_to_e4m3(float y) {
  const uint32_t u = __float_as_uint(y);
  const uint32_t sign = (u >> 24) & 0x80u;
  const uint32_t a = u & 0x7FFFFFFFu;
  uint32_t mag;
  if (a >= 0x43E00000u) {            // 448
    mag = 0x7Eu;
  } else if (a < 0x3C800000u) {      // 2^-6
    mag = (uint32_t)__builtin_rintf(__uint_as_float(a) * 512.f);
  } else {
    mag = ((a + 0x7FFFFu + ((a >> 20) & 1u)) >> 20) - (120u << 3);
  }
  return sign | mag;
}

// Bits per code of a packed tier.
__device__ __forceinline__ int tier_code_bits(int tier) {
  return tier == KV_TIER_I4 ? 4 : tier == KV_TIER_I2 ? 2 : tier == KV_TIER_B1 ? 1 : 8;
}

// Encodes one 32-element group of float32 values into packed tier `tier`.
__device__ __forceinline__ void encode_group(const float (&x)[32], int tier, uint32_t (&c)[32], float& s, float& z) {
  if (tier == KV_TIER_B1) {
    float t[16];
#pragma unroll
    for (int j = 0; j < 16; ++j) t[j] = x[2 * j] + x[2 * j + 1];
#pragma unroll
    for (int len = 8; len >= 1; len >>= 1)
#pragma unroll
      for (int j = 0; j < len; ++j) t[j] = t[2 * j] + t[2 * j + 1];
    z = f16_sat(t[0] / 32.f);
#pragma unroll
    for (int j = 0; j < 16; ++j) t[j] = fabsf(x[2 * j] - z) + fabsf(x[2 * j + 1] - z);
#pragma unroll
    for (int len = 8; len >= 1; len >>= 1)
#pragma unroll
      for (int j = 0; j < len; ++j) t[j] = t[2 * j] + t[2 * j + 1];
    s = f16_sat(t[0] / 32.f);
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = x[j] >= z ? 1u : 0u;
  } else if (tier == KV_TIER_FP8) {
    float amax = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(x[j]));
    s = f16_sat(amax / 448.f);
    z = 0.f;
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = s != 0.f ? f32_to_e4m3(x[j] / s) : 0u;
  } else {
    const int bits = tier_code_bits(tier);
    const float qmax = (float)((1 << bits) - 1);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) { mn = fminf(mn, x[j]); mx = fmaxf(mx, x[j]); }
    s = f16_sat((mx - mn) / qmax);
    z = f16_sat(mn);
#pragma unroll
    for (int j = 0; j < 32; ++j) {
      float cj = 0.f;
      if (s != 0.f) cj = fminf(fmaxf(__builtin_rintf((x[j] - z) / s), 0.f), qmax);
      c[j] = (uint32_t)cj;
    }
  }
}

// The 1-bit tier's side-table word of a group: the element farthest from z
// (float32 |x - z|, lowest index on ties) with its float16 value.
__device__ __forceinline__ uint32_t outlier_word(const float (&x)[32], float z) {
  int idx = 0;
  float best = fabsf(x[0] - z);
#pragma unroll
  for (int j = 1; j < 32; ++j) {
    const float dv = fabsf(x[j] - z);
    if (dv > best) { best = dv; idx = j; }
  }
  float v = x[0];
#pragma unroll
  for (int j = 1; j < 32; ++j) v = j == idx ? x[j] : v;
  return (uint32_t)idx | ((uint32_t)f16_bits(f16_sat(v)) << 16);
}

// Writes one encoded group: its codes (LSB first) into token row `row` of a
// code pool ([slots][Hkv][P][D*bits/8]) and its (scale, zero) pair.
template <int D>
__device__ __forceinline__ void store_group(uint8_t* codes, uint16_t* scale_zero, size_t row, int grp, int bits,
                                            const uint32_t (&c)[32], float s, float z) {
  uint32_t* dst = reinterpret_cast<uint32_t*>(codes + row * (D * bits / 8) + grp * 4 * bits);
  const int per_word = 32 / bits;
  for (int wdx = 0; wdx < bits; ++wdx) {
    uint32_t word = 0;
    for (int j = 0; j < per_word; ++j) word |= c[wdx * per_word + j] << (j * bits);
    dst[wdx] = word;
  }
  uint16_t* szp = scale_zero + (row * (D / 32) + grp) * 2;
  szp[0] = f16_bits(s);
  szp[1] = f16_bits(z);
}

template <int D, bool F16>
__global__ __launch_bounds__(256) void pack_tier_kernel(const uint16_t* __restrict__ src16,
                                                        const int32_t* __restrict__ src_pages,
                                                        const int32_t* __restrict__ dst_slots, int n,
                                                        int Hkv, int P, int tier,
                                                        uint8_t* __restrict__ codes,
                                                        uint16_t* __restrict__ scale_zero,
                                                        uint32_t* __restrict__ outliers) {
  constexpr int NG = D / 32;
  const int bits = tier_code_bits(tier);
  const size_t total = (size_t)n * Hkv * P * NG;
  for (size_t id = (size_t)blockIdx.x * blockDim.x + threadIdx.x; id < total;
       id += (size_t)gridDim.x * blockDim.x) {
    size_t r = id;
    const int grp = (int)(r % NG); r /= NG;
    const int tk = (int)(r % P); r /= P;
    const int g = (int)(r % Hkv); r /= Hkv;
    const int i = (int)r;
    const int sp = src_pages ? src_pages[i] : i;
    const int ds = dst_slots ? dst_slots[i] : i;
    const uint16_t* xs = src16 + (((size_t)sp * Hkv + g) * P + tk) * D + grp * 32;
    float x[32];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x4_t w = ld16(xs + 8 * v);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * v + 2 * j] = lo16<F16>(w[j]);
        x[8 * v + 2 * j + 1] = hi16<F16>(w[j]);
      }
    }
    uint32_t c[32];
    float s, z;
    encode_group(x, tier, c, s, z);
    const size_t row = ((size_t)ds * Hkv + g) * P + tk;
    store_group<D>(codes, scale_zero, row, grp, bits, c, s, z);
    if (outliers) outliers[row * NG + grp] = outlier_word(x, z);
  }
}

hipError_t launch_pack_tier(const kv_layout& L, const void* src16, const int32_t* src_pages, int n,
                            int tier, uint8_t* codes, void* scale_zero, uint32_t* outliers,
                            const int32_t* dst_slots, hipStream_t st) {
  const size_t total = (size_t)n * L.num_kv_heads * L.page_size * (L.head_dim / 32);
  const int blocks = (int)((total + 255) / 256 < 65536 ? (total + 255) / 256 : 65536);
  const uint16_t* s = (const uint16_t*)src16;
  uint16_t* sz = (uint16_t*)scale_zero;
  const bool f16 = L.kv_dtype == KV_F16;
  if (L.head_dim == 64) {
    if (f16) hipLaunchKernelGGL((pack_tier_kernel<64, true>), dim3(blocks), dim3(256), 0, st, s, src_pages, dst_slots, n, L.num_kv_heads, L.page_size, tier, codes, sz, outliers);
    else hipLaunchKernelGGL((pack_tier_kernel<64, false>), dim3(blocks), dim3(256), 0, st, s, src_pages, dst_slots, n, L.num_kv_heads, L.page_size, tier, codes, sz, outliers);
  } else {
    if (f16) hipLaunchKernelGGL((pack_tier_kernel<128, true>), dim3(blocks), dim3(256), 0, st, s, src_pages, dst_slots, n, L.num_kv_heads, L.page_size, tier, codes, sz, outliers);
    else hipLaunchKernelGGL((pack_tier_kernel<128, false>), dim3(blocks), dim3(256), 0, st, s, src_pages, dst_slots, n, L.num_kv_heads, L.page_size, tier, codes, sz, outliers);
  }
  return hipGetLastError();
}

// ---------------------------------------------------------------- demotion

// Re-encodes the pages a tier plan moves (ARGUS, "Visual Architecture": the
// compression cascade).  Block (i, b) takes move i of sequence b: every
// 32-element group of the page's K and V (all KV heads and tokens) is decoded
// from its current tier (page_entry) and encoded into the new one at slot
// phys, then the page's entry is switched.  Blocks past a row's move count
// exit.
struct TierPools {
  const uint16_t* k16;
  const uint16_t* v16;
  uint8_t* kq[KV_NUM_PACKED_TIERS];
  uint8_t* vq[KV_NUM_PACKED_TIERS];
  uint16_t* ksz[KV_NUM_PACKED_TIERS];
  uint16_t* vsz[KV_NUM_PACKED_TIERS];
  uint32_t* kout;
  uint32_t* vout;
};

template <int D, bool F16>
__device__ __forceinline__ void decode_group_any(const TierPools& tp, int kv, uint32_t tier, size_t row, int grp,
                                                 float (&x)[32]) {
  if (tier == KV_TIER_NATIVE) {
    const uint16_t* xs = (kv == 0 ? tp.k16 : tp.v16) + row * D + grp * 32;
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x4_t w = ld16(xs + 8 * v);
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        x[8 * v + 2 * j] = lo16<F16>(w[j]);
        x[8 * v + 2 * j + 1] = hi16<F16>(w[j]);
      }
    }
    return;
  }
  const int t = (int)tier - 1;
  const uint8_t* codes = kv == 0 ? tp.kq[t] : tp.vq[t];
  const uint16_t* sz = kv == 0 ? tp.ksz[t] : tp.vsz[t];
  switch (tier) {
    case KV_TIER_I8: decode_run<D, 32, 8>(codes, sz, row, grp * 32, x); break;
    case KV_TIER_I4: decode_run<D, 32, 4>(codes, sz, row, grp * 32, x); break;
    case KV_TIER_I2: decode_run<D, 32, 2>(codes, sz, row, grp * 32, x); break;
    case KV_TIER_FP8:
#pragma unroll
      for (int j = 0; j < 4; ++j) {
        float y[8];
        decode_fp8<D, 8>(codes, sz, row, grp * 32 + 8 * j, y);
#pragma unroll
        for (int e = 0; e < 8; ++e) x[8 * j + e] = y[e];
      }
      break;
    default: decode_run<D, 32, 1>(codes, sz, row, grp * 32, x); break;
  }
}

template <int D, bool F16>
__global__ __launch_bounds__(256) void tier_demote_kernel(TierPools tp, uint32_t* __restrict__ page_entry, int Hkv,
                                                          int P, int max_pages, const int32_t* __restrict__ moves,
                                                          const int32_t* __restrict__ move_count) {
  constexpr int NG = D / 32;
  const int i = blockIdx.x, b = blockIdx.y;
  if (i >= move_count[b]) return;
  const int32_t* mv = moves + ((size_t)b * max_pages + i) * 2;
  const int phys = mv[0], nt = mv[1];
  const uint32_t e = page_entry[phys];
  const uint32_t ot = e >> 29, oslot = e & 0x1FFFFFFFu;
  const int bits = tier_code_bits(nt);
  const int groups = 2 * Hkv * P * NG;
  for (int id = threadIdx.x; id < groups; id += 256) {
    int r = id;
    const int grp = r % NG; r /= NG;
    const int tk = r % P; r /= P;
    const int g = r % Hkv; r /= Hkv;
    const int kv = r;
    float x[32];
    decode_group_any<D, F16>(tp, kv, ot, ((size_t)oslot * Hkv + g) * P + tk, grp, x);
    uint32_t c[32];
    float s, z;
    encode_group(x, nt, c, s, z);
    const size_t nrow = ((size_t)phys * Hkv + g) * P + tk;
    store_group<D>(kv == 0 ? tp.kq[nt - 1] : tp.vq[nt - 1], kv == 0 ? tp.ksz[nt - 1] : tp.vsz[nt - 1], nrow, grp,
                   bits, c, s, z);
    if (nt == KV_TIER_B1 && tp.kout) (kv == 0 ? tp.kout : tp.vout)[nrow * NG + grp] = outlier_word(x, z);
  }
  __syncthreads();
  if (threadIdx.x == 0) page_entry[phys] = ((uint32_t)nt << 29) | (uint32_t)phys;
}

hipError_t launch_tier_demote(const kv_layout& L, const kv_pages& pg, uint32_t* page_entry, int B, int max_pages,
                              const int32_t* moves, const int32_t* move_count, hipStream_t st) {
  TierPools tp;
  tp.k16 = (const uint16_t*)pg.k16;
  tp.v16 = (const uint16_t*)pg.v16;
  for (int t = 0; t < KV_NUM_PACKED_TIERS; ++t) {
    tp.kq[t] = const_cast<uint8_t*>(pg.kq[t]);
    tp.vq[t] = const_cast<uint8_t*>(pg.vq[t]);
    tp.ksz[t] = (uint16_t*)const_cast<void*>(pg.ksz[t]);
    tp.vsz[t] = (uint16_t*)const_cast<void*>(pg.vsz[t]);
  }
  tp.kout = const_cast<uint32_t*>(pg.kout);
  tp.vout = const_cast<uint32_t*>(pg.vout);
  const dim3 grid(max_pages, B);
  const bool f16 = L.kv_dtype == KV_F16;
  if (L.head_dim == 64) {
    if (f16) hipLaunchKernelGGL((tier_demote_kernel<64, true>), grid, dim3(256), 0, st, tp, page_entry, L.num_kv_heads, L.page_size, max_pages, moves, move_count);
    else hipLaunchKernelGGL((tier_demote_kernel<64, false>), grid, dim3(256), 0, st, tp, page_entry, L.num_kv_heads, L.page_size, max_pages, moves, move_count);
  } else {
    if (f16) hipLaunchKernelGGL((tier_demote_kernel<128, true>), grid, dim3(256), 0, st, tp, page_entry, L.num_kv_heads, L.page_size, max_pages, moves, move_count);
    else hipLaunchKernelGGL((tier_demote_kernel<128, false>), grid, dim3(256), 0, st, tp, page_entry, L.num_kv_heads, L.page_size, max_pages, moves, move_count);
  }
  return hipGetLastError();
}

}  // namespace kvs
