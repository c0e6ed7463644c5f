"""Pins for the packed-tier codec (CPU only).

Hand-worked bytes and groups (tests/golden/), exactly representable inputs,
the rounding rule at an exact tie, the per-group error bound and the 1-bit
value set.
"""

import json
import os

import numpy as np

from oracle.codec import (
    BITS_OF_TIER, TIER_I8, TIER_I4, TIER_I2, TIER_B1,
    encode_group_int, encode_group_1bit, encode_vector, decode_vector,
    pack_codes, unpack_codes, _tree_sum,
)
from oracle.rounding import round_bf16

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_golden_bytes():
    g = json.load(open(os.path.join(GOLDEN, "codec_bytes.json")))
    for case in g["cases"]:
        codes = np.array(case["codes"], dtype=np.uint8)
        packed = pack_codes(codes, case["bits"])
        assert list(packed) == case["bytes"], case
        assert list(unpack_codes(packed, case["bits"], len(codes))) == case["codes"]


def test_golden_int4_ramp():
    g = json.load(open(os.path.join(GOLDEN, "int4_ramp.json")))
    x = np.array(g["x"], dtype=np.float32)
    c, s, z = encode_group_int(x, 4)
    assert float(s) == g["scale"] and float(z) == g["zero"]
    assert list(c) == g["codes"]
    xh = decode_vector(pack_codes(c, 4), np.array([[s, z]]), TIER_I4, 32)
    assert np.max(np.abs(xh - x)) == g["max_abs_error"]


def test_round_half_to_even_at_exact_tie():
    # group min 0, max 15 -> s = 1, z = 0; 2.5 and 3.5 sit exactly between codes
    x = np.zeros(32, dtype=np.float32)
    x[1] = 15.0
    x[2] = 2.5
    x[3] = 3.5
    c, s, z = encode_group_int(x, 4)
    assert s == 1.0 and z == 0.0
    assert c[2] == 2 and c[3] == 4


def test_exactly_representable_groups_round_trip():
    rng = np.random.default_rng(0)
    for bits, s, z in [(8, 2.0 ** -6, -2.0), (4, 2.0 ** -3, -1.0), (2, 0.5, 0.25)]:
        qmax = 2 ** bits - 1
        for _ in range(50):
            c = rng.integers(0, qmax + 1, 32)
            c[rng.integers(0, 32)] = 0
            c[rng.integers(0, 32)] = qmax
            if c.min() != 0 or c.max() != qmax:
                continue
            x = (z + c * s).astype(np.float32)
            assert np.array_equal(round_bf16(x.astype(np.float64)), x)    # a 16-bit input
            cc, ss, zz = encode_group_int(x, bits)
            assert ss == s and zz == z
            np.testing.assert_array_equal(cc, c)


def test_constant_group_has_zero_scale():
    x = np.full(32, 0.75, dtype=np.float32)
    for bits in (8, 4, 2):
        c, s, z = encode_group_int(x, bits)
        assert s == 0 and z == 0.75 and not c.any()
    c, s, z = encode_group_1bit(x)
    assert z == 0.75 and s == 0 and c.all()


def test_error_bound_random_groups():
    rng = np.random.default_rng(1)
    x = round_bf16(rng.standard_normal((2000, 32)) * rng.uniform(0.01, 30, (2000, 1))).astype(np.float32)
    for bits in (8, 4, 2):
        qmax = 2 ** bits - 1
        c, s, z = encode_group_int(x, bits)
        assert c.max() <= qmax
        xh = c.astype(np.float64) * s[:, None] + z[:, None]
        mn, mx = x.min(1).astype(np.float64), x.max(1).astype(np.float64)
        bound = (s / 2 + np.maximum(0, z - mn) + np.maximum(0, mx - (z + qmax * s.astype(np.float64)))
                 + np.spacing(np.abs(x).max(1)))
        err = np.abs(xh - x).max(1)
        assert np.all(err <= bound), (bits, np.max(err - bound))
        # the quantizer must actually use its range: error well below the group range
        assert np.all(err <= (mx - mn) / qmax)


def test_one_bit_values_and_signs():
    rng = np.random.default_rng(2)
    x = round_bf16(rng.standard_normal((500, 32))).astype(np.float32)
    c, s, z = encode_group_1bit(x)
    np.testing.assert_array_equal(c, (x >= z[:, None]).astype(np.uint8))
    xh = np.where(c == 1, z[:, None] + s[:, None], z[:, None] - s[:, None])
    # z is the group mean and s the mean absolute deviation, each to float16 precision
    assert np.all(np.abs(z - x.astype(np.float64).mean(1)) <= 1e-3 * (1 + np.abs(x).max(1)))
    mad = np.abs(x - z[:, None]).astype(np.float64).mean(1)
    assert np.all(np.abs(s - mad) <= 2e-3 * mad + 1e-7)
    # hand example: +-1 halves
    y = np.array([1.0] * 16 + [-1.0] * 16, dtype=np.float32)
    cy, sy, zy = encode_group_1bit(y)
    assert zy == 0 and sy == 1 and list(cy) == [1] * 16 + [0] * 16
    packed, sz = encode_vector(y[None], TIER_B1)
    np.testing.assert_array_equal(decode_vector(packed, sz, TIER_B1, 32)[0], y)


def test_tree_sum_order_hand_example():
    # pairwise: (1 + 2^-24) -> 1, (2^-24 + 2^-24) = 2^-23, then 1 + 2^-23; left to right gives 1
    v = np.zeros(32, dtype=np.float32)
    v[0], v[1], v[2], v[3] = 1.0, 2.0 ** -24, 2.0 ** -24, 2.0 ** -24
    assert _tree_sum(v) == np.float32(1.0 + 2.0 ** -23)


def test_pack_unpack_identity_and_sizes():
    rng = np.random.default_rng(3)
    for tier, bits in BITS_OF_TIER.items():
        c = rng.integers(0, 2 ** bits, (7, 128)).astype(np.uint8)
        p = pack_codes(c, bits)
        assert p.shape == (7, 128 * bits // 8)
        np.testing.assert_array_equal(unpack_codes(p, bits, 128), c)


def test_vector_round_trip_matches_group_encoders():
    rng = np.random.default_rng(4)
    x = round_bf16(rng.standard_normal((3, 16, 128))).astype(np.float32)
    for tier in (TIER_I8, TIER_I4, TIER_I2, TIER_B1):
        packed, sz = encode_vector(x, tier)
        assert sz.shape == (3, 16, 4, 2)
        g = x.reshape(3, 16, 4, 32)
        if tier == TIER_B1:
            c, s, z = encode_group_1bit(g)
        else:
            c, s, z = encode_group_int(g, BITS_OF_TIER[tier])
        np.testing.assert_array_equal(sz[..., 0], s)
        np.testing.assert_array_equal(sz[..., 1], z)
        xh = decode_vector(packed, sz, tier, 128)
        ref = (c * s[..., None].astype(np.float64) + z[..., None] if tier != TIER_B1
               else z[..., None] + (2.0 * c - 1) * s[..., None])
        np.testing.assert_array_equal(xh, ref.reshape(3, 16, 128).astype(np.float32))
