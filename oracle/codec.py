"""Packed low-bit page tiers: encoder, decoder and byte layout (test infrastructure only).

ARGUS (argus_cache 0.1.7.1 project page), section "Visual Architecture" and the
tier legend under "Heatmap & Telemetry Legend": tiers INT8, INT4 ("2-way
bit-packed"), INT2 ("4-way bit-packed") and 1-bit ("8-way sign-packed"), and
section "Why It Works: Storage vs. Computation": packed pages are rebuilt in
high precision on chip just before attention, never used in low-bit math.
The page names bit widths and packing ratios only; everything below is a
stated reading.

Grouping: each token's K or V vector is cut into groups of 32 consecutive
head-dim elements; every group stores a float16 (scale s, zero z) pair.

Encoder, step-exact in IEEE float32 with every operation correctly rounded and
no fused multiply-add (x is the float32 value of the 16-bit input, exact):
  int-b (b = 8, 4, 2):
    mn = min x, mx = max x
    s  = fp16(fp32(mx - mn) / fp32(2^b - 1))
    z  = fp16(mn)
    c  = 0 if s == 0 else clamp(rint_even(fp32(x - z) / s), 0, 2^b - 1)
  1-bit:
    z  = fp16(T(x) / 32),  s = fp16(T(|x - z|) / 32),  c = (x >= z)
    where T is the pairwise tree sum (level by level, pairs (2i, 2i+1)).
  fp16() rounds to nearest even and saturates at +-65504.
Decoder: int-b x^ = c*s + z; 1-bit x^ = z + (2c - 1)*s.  Both are exact in
float64 for float16 s, z and b <= 8, and are returned rounded once to float32.
Byte layout, LSB first in head-dim order: int8 one code per byte; int4 element
2i in bits 0-3 and 2i+1 in bits 4-7; int2 element 4i+j in bits 2j..2j+1; 1-bit
element 8i+j in bit j.  A vector's d*b/8 code bytes are contiguous; the
(s, z) pairs live in a separate array.

FP8 tier (the cascade's first step below 16 bits, "gentle precision
quantization" in the tier legend; the page names no format).  Reading: the
OCP 8-bit float E4M3 in its finite variant (1 sign, 4 exponent bits with bias
7, 3 mantissa bits; no infinities; exponent 15 with mantissa 7 is NaN, so the
largest finite value is 448), one code per byte, with a symmetric per-group
scale so that any 16-bit input range fits:
    s = fp16(fp32(max |x|) / 448),  z = 0
    c = 0 if s == 0 else E4M3(fp32(x / s))
where E4M3(y) is the nearest finite E4M3 value to y, ties to the even code,
|y| >= 448 saturating to 448, the sign taken from y's sign bit.  Decoder: the
code's value times s plus z (exact in float64, returned as float32).

1-bit outlier side table (the tier legend: the 1-bit tier is sign-packed
"with FP16 outlier preservation"; count and format unstated).  Reading: per
32-element group, after the 1-bit encoding above (s and z unchanged), the
element e* with the largest fp32(|x_e - z|) (ties: lowest index) is kept as
v = fp16(x_e*) (round to nearest even, saturating), in one 32-bit side-table
word per group: e* in bits 0..4, the float16 bits of v in bits 16..31.  The
decoder returns v at e* and z +- s elsewhere.

Pinned in tests/test_oracle_codec.py: hand-packed bytes (0xA3, 0xE4, 0x8D), the
int4 ramp 0..31 (s = fp16(31/15) = 2.06640625), exactly representable inputs
mapping back to their codes, the per-group error bound, the 1-bit value set
and sign, and pack/unpack identity.  FP8 in tests/test_oracle_fp8.py: the
format's landmark codes, torch's float8_e4m3fn cast for in-range values, a
brute-force nearest-value search over all 127 magnitudes, a hand-worked group
(tests/golden/fp8_group.json), the relative error bound and saturation.
Outlier words in tests/test_oracle_outlier.py: a hand-worked group, ties,
exactness of the kept element, the rest of the group unchanged, saturation.
"""

import numpy as np

from .rounding import round_fp16_sat

TIER_NATIVE, TIER_I8, TIER_I4, TIER_I2, TIER_B1, TIER_FP8 = 0, 1, 2, 3, 4, 5
BITS_OF_TIER = {TIER_I8: 8, TIER_I4: 4, TIER_I2: 2, TIER_B1: 1, TIER_FP8: 8}
FP8_MAX = 448.0
GROUP = 32


def _f16(x32):
    return round_fp16_sat(x32).astype(np.float32)


def encode_group_int(x, bits):
    """x: float32 (..., 32).  Returns (codes uint8 (..., 32), s f32 (...), z f32 (...))."""
    x = np.asarray(x, dtype=np.float32)
    qmax = np.float32(2 ** bits - 1)
    mn = x.min(axis=-1)
    mx = x.max(axis=-1)
    with np.errstate(over="ignore"):
        s = _f16((mx - mn) / qmax)
    z = _f16(mn)
    with np.errstate(divide="ignore", invalid="ignore"):
        c = np.rint((x - z[..., None]) / s[..., None])
    c = np.clip(c, np.float32(0), qmax)
    c = np.where((s == 0)[..., None], np.float32(0), c)
    return c.astype(np.uint8), s, z


def _tree_sum(v):
    v = np.asarray(v, dtype=np.float32)
    while v.shape[-1] > 1:
        v = v[..., 0::2] + v[..., 1::2]
    return v[..., 0]


def encode_group_1bit(x):
    """x: float32 (..., 32).  Returns (codes uint8 in {0,1}, s, z)."""
    x = np.asarray(x, dtype=np.float32)
    n = np.float32(GROUP)
    z = _f16(_tree_sum(x) / n)
    s = _f16(_tree_sum(np.abs(x - z[..., None])) / n)
    c = (x >= z[..., None]).astype(np.uint8)
    return c, s, z


def e4m3_magnitudes():
    """float64 values of the non-negative finite E4M3 codes 0..126 (ascending):
    exponent field e = code >> 3, mantissa m = code & 7; e = 0 is subnormal,
    m * 2^-9, otherwise 2^(e - 7) * (1 + m / 8)."""
    code = np.arange(127)
    e, m = code >> 3, code & 7
    return np.where(e == 0, m * 2.0 ** -9, np.ldexp(1.0 + m / 8.0, e - 7))


def e4m3_value(code):
    """float64 value of E4M3 codes (bit 7 = sign); code 0x7F / 0xFF (NaN) never occurs."""
    c = np.asarray(code, dtype=np.int64)
    mag = e4m3_magnitudes()[c & 0x7F]
    return np.where((c & 0x80) != 0, -mag, mag)


def round_e4m3(y):
    """float32 y -> E4M3 code (uint8): nearest finite magnitude, ties to the even
    code, saturating at 448; sign bit copied from y."""
    y = np.asarray(y, dtype=np.float32)
    a = np.abs(y).astype(np.float64)
    vals = e4m3_magnitudes()
    hi = np.minimum(np.searchsorted(vals, a, side="left"), 126)   # first magnitude >= a (or the largest)
    lo = np.maximum(hi - 1, 0)
    d_lo, d_hi = a - vals[lo], vals[hi] - a
    mag = np.where(d_lo < d_hi, lo, np.where(d_hi < d_lo, hi, np.where(lo % 2 == 0, lo, hi)))
    return (mag | np.where(np.signbit(y), 0x80, 0)).astype(np.uint8)


def encode_group_fp8(x):
    """x: float32 (..., 32).  Returns (codes uint8 (..., 32), s f32 (...), z f32 (...))."""
    x = np.asarray(x, dtype=np.float32)
    amax = np.abs(x).max(axis=-1)
    s = _f16(amax / np.float32(FP8_MAX))
    z = np.zeros_like(s)
    with np.errstate(divide="ignore", invalid="ignore"):
        y = x / s[..., None]
    c = round_e4m3(np.where((s == 0)[..., None], np.float32(0), y))
    return c, s, z


def outlier_words(x, z):
    """Side-table words of 1-bit groups: x float32 (..., 32), z (...) their zeros."""
    x = np.asarray(x, dtype=np.float32)
    dev = np.abs(x - np.asarray(z, dtype=np.float32)[..., None])      # float32 steps
    idx = np.argmax(dev, axis=-1)                                     # first maximum
    v = np.take_along_axis(x, idx[..., None], axis=-1)[..., 0]
    bits = round_fp16_sat(v).astype(np.float16).view(np.uint16).astype(np.uint32)
    return (idx.astype(np.uint32) | (bits << np.uint32(16))).astype(np.uint32)


def apply_outliers(xh, words):
    """Decoded 1-bit groups xh float32 (..., 32) with their side-table words applied."""
    xh = np.array(xh, dtype=np.float32)
    w = np.asarray(words, dtype=np.uint32)
    idx = (w & np.uint32(31)).astype(np.int64)
    v = (w >> np.uint32(16)).astype(np.uint16).view(np.float16).astype(np.float32)
    np.put_along_axis(xh, idx[..., None], v[..., None], axis=-1)
    return xh


def pack_codes(codes, bits):
    """codes uint8 (..., d) -> bytes uint8 (..., d*bits/8), LSB first."""
    c = np.asarray(codes, dtype=np.uint8)
    if bits == 8:
        return c.copy()
    per = 8 // bits
    out = np.zeros(c.shape[:-1] + (c.shape[-1] // per,), dtype=np.uint8)
    for j in range(per):
        out |= (c[..., j::per] << (bits * j)).astype(np.uint8)
    return out


def unpack_codes(packed, bits, d):
    """Inverse of pack_codes."""
    b = np.asarray(packed, dtype=np.uint8)
    if bits == 8:
        return b.copy()
    per = 8 // bits
    mask = (1 << bits) - 1
    out = np.zeros(b.shape[:-1] + (d,), dtype=np.uint8)
    for j in range(per):
        out[..., j::per] = (b >> (bits * j)) & mask
    return out


def encode_vector(x16, tier, outliers=False):
    """Encode token vectors.

    x16: float32 (..., d) holding exact 16-bit values, d a multiple of 32.
    Returns (packed bytes (..., d*bits/8), scale_zero float32 (..., d/32, 2)),
    and for the 1-bit tier with outliers=True also the side-table words
    (..., d/32) uint32.
    """
    x = np.asarray(x16, dtype=np.float32)
    d = x.shape[-1]
    g = x.reshape(x.shape[:-1] + (d // GROUP, GROUP))
    bits = BITS_OF_TIER[tier]
    if tier == TIER_B1:
        c, s, z = encode_group_1bit(g)
    elif tier == TIER_FP8:
        c, s, z = encode_group_fp8(g)
    else:
        c, s, z = encode_group_int(g, bits)
    packed = pack_codes(c.reshape(x.shape), bits)
    if outliers and tier == TIER_B1:
        return packed, np.stack([s, z], axis=-1), outlier_words(g, z)
    return packed, np.stack([s, z], axis=-1)


def decode_vector(packed, scale_zero, tier, d, outlier=None):
    """Decode token vectors to float32 (..., d) (exact float64 value rounded once);
    outlier: the 1-bit tier's side-table words (..., d/32), applied if given."""
    bits = BITS_OF_TIER[tier]
    c = unpack_codes(packed, bits, d)
    c = e4m3_value(c) if tier == TIER_FP8 else c.astype(np.float64)
    sz = np.asarray(scale_zero, dtype=np.float64)
    c = c.reshape(c.shape[:-1] + (d // GROUP, GROUP))
    s = sz[..., 0][..., None]
    z = sz[..., 1][..., None]
    if tier == TIER_B1:
        xh = z + (2.0 * c - 1.0) * s
    else:
        xh = c * s + z
    xh = xh.astype(np.float32)
    if outlier is not None and tier == TIER_B1:
        xh = apply_outliers(xh, outlier)
    return xh.reshape(xh.shape[:-2] + (d,))
