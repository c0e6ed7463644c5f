"""Pins for group aggregation and top-k selection (CPU only)."""

import math

import numpy as np

from oracle.select import group_aggregate, selection_count, select_pages


def test_aggregate_is_a_log_distribution():
    rng = np.random.default_rng(0)
    for G in [1, 4, 8]:
        s = rng.standard_normal((G, 300)) * 3 + 5
        S = group_aggregate(s)
        assert abs(np.exp(S).sum() - 1.0) <= 1e-12
        assert np.all(S <= 0)


def test_aggregate_g1_is_the_score_order():
    rng = np.random.default_rng(1)
    s = rng.standard_normal((1, 500))
    S = group_aggregate(s)
    lse = np.log(np.exp(s[0]).sum())
    np.testing.assert_allclose(S, s[0] - lse, atol=1e-12)
    assert list(np.argsort(-S, kind="stable")) == list(np.argsort(-s[0], kind="stable"))


def test_aggregate_mean_of_fractions_brute_force():
    rng = np.random.default_rng(2)
    s = rng.standard_normal((4, 7))
    frac = np.exp(s) / np.exp(s).sum(axis=1, keepdims=True)
    np.testing.assert_allclose(np.exp(group_aggregate(s)), frac.mean(0), rtol=1e-12)


def test_selection_count():
    assert selection_count(2048, 0.08) == 164
    assert selection_count(4096, 0.10) == 410
    assert selection_count(8192, 0.05) == 410
    assert selection_count(64, 0.125) == 8
    assert selection_count(64, 0.0, k_fixed=8) == 8
    assert selection_count(5, 0.0, k_fixed=8) == 5
    assert selection_count(10, 1e-9) == 1
    assert selection_count(0, 0.5) == 0
    assert selection_count(3, 2.0) == 3
    # keep is a float32 value: 0.1f * 10 = 1.0000000149... -> 2
    assert selection_count(10, 0.1) == 2


def _brute(S, k, ff, fl):
    npg = len(S)
    key = []
    for p in range(npg):
        v = S[p]
        if p < ff or p >= npg - fl:
            v = math.inf
        elif math.isnan(v):
            v = -math.inf
        key.append((-v, p))
    return sorted(p for _, p in sorted(key)[:k])


def test_selection_brute_force_tiny():
    rng = np.random.default_rng(3)
    for trial in range(10000):
        npg = int(rng.integers(1, 13))
        if trial % 3 == 0:
            S = rng.integers(-3, 1, npg).astype(np.float64)       # many ties
        else:
            S = rng.standard_normal(npg)
        if trial % 7 == 0:
            S[rng.integers(0, npg)] = np.nan
        k = int(rng.integers(1, npg + 1))
        ff = int(rng.integers(0, 3)) if trial % 5 == 0 else 0
        fl = int(rng.integers(0, 3)) if trial % 11 == 0 else 0
        got = list(select_pages(S, k, ff, fl))
        assert got == _brute(list(S), k, ff, fl), (S, k, ff, fl)


def test_constant_and_nan_scores_pick_lowest_indices():
    assert list(select_pages(np.full(20, -3.0), 5)) == [0, 1, 2, 3, 4]
    assert list(select_pages(np.full(20, np.nan), 3)) == [0, 1, 2]
    S = np.full(10, np.nan)
    S[7] = -100.0
    assert list(select_pages(S, 2)) == [0, 7]


def test_forced_pages_count_towards_k():
    S = np.linspace(0, -1, 12)
    assert list(select_pages(S, 4, n_force_first=1, n_force_last=2)) == [0, 1, 10, 11]
    assert list(select_pages(S, 2, n_force_first=3)) == [0, 1]
