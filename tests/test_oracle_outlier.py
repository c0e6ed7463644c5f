"""Pins of the oracle's 1-bit outlier side table: a hand-worked group, ties,
exactness of the preserved element, the rest of the group unchanged,
saturation."""

import numpy as np

import oracle


def test_hand_worked_group():
    x = np.array([0.5] * 31 + [7.0], dtype=np.float32)
    packed, sz, words = oracle.encode_vector(x, oracle.TIER_B1, outliers=True)
    # z = fp16(22.5 / 32) = 0.703125; |7 - z| = 6.296875 is the largest deviation
    assert sz[0, 1] == np.float32(0.703125)
    assert words.tolist() == [31 | (0x4700 << 16)]                 # fp16(7.0) = 0x4700
    xh = oracle.decode_vector(packed, sz, oracle.TIER_B1, 32, outlier=words)
    assert xh[31] == 7.0
    plain = oracle.decode_vector(packed, sz, oracle.TIER_B1, 32)
    np.testing.assert_array_equal(xh[:31], plain[:31])


def test_ties_take_the_lowest_index():
    x = np.array([1.0, -1.0] * 16, dtype=np.float32)
    _, sz, words = oracle.encode_vector(x, oracle.TIER_B1, outliers=True)
    assert sz[0, 1] == 0.0 and (words[0] & 31) == 0
    assert (words[0] >> 16) == 0x3C00                              # fp16(1.0)


def test_preserved_element_is_exact_and_error_not_larger():
    rng = np.random.default_rng(11)
    x = oracle.round_bf16(rng.standard_normal((200, 128)) * np.exp2(rng.uniform(-3, 3, (200, 1))))
    x = x.astype(np.float32)
    packed, sz, words = oracle.encode_vector(x, oracle.TIER_B1, outliers=True)
    with_o = oracle.decode_vector(packed, sz, oracle.TIER_B1, 128, outlier=words)
    without = oracle.decode_vector(packed, sz, oracle.TIER_B1, 128)
    g = x.reshape(200, 4, 32)
    idx = (words & 31).astype(np.int64)
    kept = np.take_along_axis(with_o.reshape(200, 4, 32), idx[..., None], -1)[..., 0]
    orig = np.take_along_axis(g, idx[..., None], -1)[..., 0]
    np.testing.assert_array_equal(kept, orig)                        # bf16 values in fp16 range are exact
    err_o = np.abs(with_o - x).reshape(200, 4, 32).max(-1)
    err = np.abs(without - x).reshape(200, 4, 32).max(-1)
    assert np.all(err_o <= err)
    # the element taken is the largest deviation from z
    z = sz[..., 1]
    dev = np.abs(g - z[..., None].astype(np.float32))
    np.testing.assert_array_equal(idx, np.argmax(dev, -1))


def test_saturation():
    x = np.zeros(32, dtype=np.float32)
    x[5] = 1.0e5
    _, _, words = oracle.encode_vector(x, oracle.TIER_B1, outliers=True)
    assert (words[0] & 31) == 5 and (words[0] >> 16) == 0x7BFF      # 65504
