"""Pins of the oracle's tier demotion (compression cascade): a hand-worked
sequence of calls, convergence to the budgets, agreement with top-k selection
at every cumulative budget, the cascade invariants and the chained codec."""

import numpy as np
import pytest

import oracle

NAT, FP8, I8, I4, I2, B1 = 0, 5, 1, 2, 3, 4


def test_hand_worked_calls():
    # 6 pages; budgets: 1 native, 1 FP8, 1 int8, 1 int4, 1 int2, the rest 1-bit
    imp = [0.1, 5.0, 2.0, -1.0, 4.0, 3.0]
    # ranks: page 1 (5.0), 4 (4.0), 5 (3.0), 2 (2.0), 0 (0.1), 3 (-1.0)
    # desired levels: p1 0, p4 1, p5 2, p2 3, p0 4, p3 5
    caps = [1, 1, 1, 1, 1]
    t = np.array([NAT] * 6)
    t = oracle.plan_row(imp, t, caps)
    assert t.tolist() == [FP8, NAT, FP8, FP8, FP8, FP8]          # everyone but p1 steps once
    t = oracle.plan_row(imp, t, caps)
    assert t.tolist() == [I8, NAT, I8, I8, FP8, I8]             # p4 has reached level 1
    t = oracle.plan_row(imp, t, caps)
    assert t.tolist() == [I4, NAT, I4, I4, FP8, I8]
    for _ in range(5):
        t = oracle.plan_row(imp, t, caps)
    assert t.tolist() == [I2, NAT, I4, B1, FP8, I8]             # every page at its desired level
    # a page that becomes important again is not promoted
    imp2 = [9.0, 5.0, 2.0, -1.0, 4.0, 3.0]
    t2 = oracle.plan_row(imp2, t, caps)
    assert t2[0] == I2                                          # stays, never promoted
    # forced pages (sink first, newest last) outrank any importance
    t3 = oracle.plan_row(imp, np.array([NAT] * 6), caps, n_force_first=1, n_force_last=1)
    assert t3[0] == NAT and t3[5] == FP8 and t3[1] == FP8       # ranks: p0, p5, then p1 ...


def test_importance_is_max_over_heads_nan_low():
    S = np.array([[0.0, np.nan, -3.0], [1.0, -2.0, np.nan]])
    np.testing.assert_array_equal(oracle.page_importance(S), [1.0, -2.0, -3.0])
    S = np.array([[np.nan, np.nan]])
    assert np.all(oracle.page_importance(S) == -np.inf)


@pytest.mark.parametrize("seed", range(20))
def test_desired_levels_follow_top_k_at_every_budget(seed):
    rng = np.random.default_rng(seed)
    npg = int(rng.integers(1, 60))
    imp = rng.standard_normal(npg)
    imp[rng.random(npg) < 0.2] = 0.5                            # ties
    imp[rng.random(npg) < 0.05] = np.nan
    caps = rng.integers(0, 8, 5)
    ff, fl = int(rng.integers(0, 3)), int(rng.integers(0, 2))
    d = oracle.desired_levels(oracle.rank_pages(np.where(np.isnan(imp), -np.inf, imp), ff, fl), caps)
    bound = 0
    for lvl in range(5):
        bound += int(caps[lvl])
        k = min(bound, npg)
        top = set(oracle.select_pages(imp, k, ff, fl).tolist())
        assert set(np.nonzero(d <= lvl)[0].tolist()) == top, (lvl, k)


@pytest.mark.parametrize("seed", range(10))
def test_cascade_invariants_and_convergence(seed):
    rng = np.random.default_rng(100 + seed)
    npg = int(rng.integers(5, 80))
    caps = rng.integers(0, 10, 5)
    tiers = np.array(oracle.TIER_OF_LEVEL)[rng.integers(0, 3, npg)]
    imp = rng.standard_normal(npg)
    for call in range(7):
        new = oracle.plan_row(imp, tiers, caps)
        lo = np.array([oracle.LEVEL_OF_TIER[int(t)] for t in tiers])
        ln = np.array([oracle.LEVEL_OF_TIER[int(t)] for t in new])
        assert np.all((ln == lo) | (ln == lo + 1))              # one step at most, never up
        tiers = new
    # after enough calls every page holds max(start, desired): budgets are met exactly when
    # every page started at or above its desired level
    fresh = np.array([NAT] * npg)
    for _ in range(6):
        fresh = oracle.plan_row(imp, fresh, caps)
    levels = np.array([oracle.LEVEL_OF_TIER[int(t)] for t in fresh])
    rem = npg
    for lvl in range(5):
        want = min(int(caps[lvl]), rem)
        assert np.sum(levels == lvl) == want
        rem -= want
    assert np.sum(levels == 5) == rem


def test_chained_codec_consistency_and_bounds():
    rng = np.random.default_rng(5)
    x16 = oracle.round_bf16(rng.standard_normal((40, 128))).astype(np.float32)
    # native -> FP8 re-encodes the 16-bit values themselves
    p1, sz1 = oracle.retier_vectors(x16, NAT, FP8, 128)
    q1, qz1 = oracle.encode_vector(x16, FP8)
    np.testing.assert_array_equal(p1, q1)
    np.testing.assert_array_equal(sz1, qz1)
    # each further step encodes the previous step's decoded values, within that tier's bound
    x, tier = oracle.decode_vector(p1, sz1, FP8, 128), FP8
    for nxt in (I8, I4, I2, B1):
        p, sz = oracle.retier_vectors(x, tier, nxt, 128)
        xh = oracle.decode_vector(p, sz, nxt, 128)
        g = x.reshape(40, 4, 32).astype(np.float64)
        gh = xh.reshape(40, 4, 32).astype(np.float64)
        s = sz[..., 0][..., None].astype(np.float64)
        if nxt == B1:
            # 1-bit keeps the group mean's sign split: every value is z +- s
            z = sz[..., 1][..., None].astype(np.float64)
            assert np.all(np.isclose(np.abs(gh - z), s, rtol=0, atol=1e-6 * (1 + np.abs(z))))
        else:
            assert np.all(np.abs(gh - g) <= 0.5 * s + 1e-6 * np.abs(g) + 1e-30)
        x, tier = xh, nxt
    with pytest.raises(AssertionError):
        oracle.retier_vectors(x16, I8, FP8, 128)                  # no promotion
