"""Pins of the oracle's FP8 (E4M3) tier against what the format and the
mathematics fix: the format's landmark values, torch's float8_e4m3fn cast (an
independent implementation) for in-range values, a brute-force nearest-value
search, a hand-worked group, the error bound and saturation."""

import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "fp8_group.json")


def test_format_landmarks():
    v = oracle.e4m3_magnitudes()
    assert v.shape == (127,) and np.all(np.diff(v) > 0)
    assert v[0x00] == 0.0
    assert v[0x01] == 2.0 ** -9              # smallest subnormal
    assert v[0x07] == 7 * 2.0 ** -9          # largest subnormal
    assert v[0x08] == 2.0 ** -6              # smallest normal
    assert v[0x38] == 1.0
    assert v[0x7E] == 448.0 == oracle.FP8_MAX
    assert oracle.e4m3_value(0xB8) == -1.0 and oracle.e4m3_value(0xFE) == -448.0


def _probe_values(rng, n):
    """float32 values over the whole E4M3 range: random, exact codes, and the
    exact midpoints between neighbouring codes (the ties)."""
    v = oracle.e4m3_magnitudes()
    mids = (v[:-1] + v[1:]) / 2
    rnd = np.exp2(rng.uniform(-12, 8.8, n)) * rng.choice([-1, 1], n)
    return np.concatenate([rnd, v, -v, mids, -mids, [0.0, -0.0]]).astype(np.float32)


def test_matches_torch_cast_in_range():
    y = _probe_values(np.random.default_rng(7), 20000)
    y = y[np.abs(y) <= 448]
    ours = oracle.round_e4m3(y)
    theirs = torch.from_numpy(y).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(ours, theirs)


def test_brute_force_nearest_even():
    v = oracle.e4m3_magnitudes()
    y = _probe_values(np.random.default_rng(8), 400)
    got = oracle.round_e4m3(y)
    for yi, ci in zip(y, got):
        a = abs(float(yi))
        best, best_d = None, None
        for code in range(127):
            d = abs(v[code] - a)
            if best is None or d < best_d or (d == best_d and code % 2 == 0):
                best, best_d = code, d
        if a >= 448:
            best = 0x7E
        want = best | (0x80 if np.signbit(yi) else 0)
        assert ci == want, (yi, hex(ci), hex(want))


def test_saturation():
    y = np.array([448.0, 460.0, 464.0, 465.0, 1e6, 3e38, -500.0], dtype=np.float32)
    np.testing.assert_array_equal(oracle.round_e4m3(y), [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE])


def test_hand_worked_groups():
    g = json.load(open(GOLDEN))
    x = np.array(g["group1_x"], dtype=np.float32)
    assert np.array_equal(oracle.round_bf16(x.astype(np.float64)), x)          # exact bf16 inputs
    c, s, z = oracle.encode_group_fp8(x)
    assert float(s) == g["group1_s"] and float(z) == 0.0
    assert [int(h, 16) for h in g["group1_codes"]] == c.tolist()
    x2 = np.zeros(32, dtype=np.float32)
    x2[:3] = g["group2_x_head"]
    assert np.array_equal(x2.astype(np.float16).astype(np.float32), x2)        # exact fp16 inputs
    c2, s2, _ = oracle.encode_group_fp8(x2)
    assert float(s2) == g["group2_s"]
    assert [int(h, 16) for h in g["group2_codes_head"]] == c2[:3].tolist()


def test_error_bound_and_round_trip():
    rng = np.random.default_rng(9)
    x = (rng.standard_normal((500, 4, 128)) * np.exp2(rng.uniform(-8, 8, (500, 4, 1)))).astype(np.float32)
    x = oracle.round_bf16(x.astype(np.float64)).astype(np.float32)
    packed, sz = oracle.encode_vector(x, oracle.TIER_FP8)
    assert packed.shape == x.shape and packed.dtype == np.uint8
    xh = oracle.decode_vector(packed, sz, oracle.TIER_FP8, 128)
    s = np.repeat(sz[..., 0], 32, axis=-1).astype(np.float64)
    err = np.abs(xh.astype(np.float64) - x)
    assert np.all(err <= (2.0 ** -4 + 2.0 ** -23) * np.abs(x) + s * 2.0 ** -10)
    assert np.all(sz[..., 1] == 0)
    # values that are exactly code * s decode to themselves and re-encode to the same codes
    p2, sz2 = oracle.encode_vector(xh, oracle.TIER_FP8)
    np.testing.assert_array_equal(sz2, sz)
    np.testing.assert_array_equal(p2, packed)
    # max |x| of a group maps to (nearly) 448 and never exceeds it
    assert np.all(np.abs(oracle.e4m3_value(packed)) <= 448)


@pytest.mark.parametrize("scale", [0.0, 1e-30])
def test_degenerate_groups(scale):
    x = np.full((1, 32), scale, dtype=np.float32)
    c, s, z = oracle.encode_group_fp8(x)
    assert float(s[0]) == 0.0 and np.all(c == 0)
    assert np.all(oracle.decode_vector(c, np.stack([s, z], -1)[:, None], oracle.TIER_FP8, 32) == 0)
