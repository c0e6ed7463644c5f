"""Pins for group aggregation and top-k selection (CPU only)."""

import math

import numpy as np

from oracle.select import group_aggregate, selection_count, select_pages, coverage_count


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


# ---------------------------------------------------------------- coverage mode

def _brute_coverage(S, coverage, k_cap, ff=0, fl=0):
    npg = len(S)
    if npg == 0:
        return 0
    items = []
    n_forced = 0
    for p in range(npg):
        v = S[p]
        m = 0.0 if math.isnan(v) else min(math.exp(v), 1.0)
        if p < ff or p >= npg - fl:
            key = math.inf
            n_forced += 1
        elif math.isnan(v):
            key = -math.inf
        else:
            key = v
        items.append((-key, p, m))
    items.sort()
    total, k = 0.0, npg
    for i, (_, _, m) in enumerate(items):
        total += m
        if total >= coverage:
            k = i + 1
            break
    return min(max(k, n_forced, 1), k_cap, npg)


def test_coverage_count_brute_force_tiny():
    rng = np.random.default_rng(11)
    for trial in range(5000):
        npg = int(rng.integers(1, 13))
        x = rng.standard_normal(npg) * 2
        if trial % 3 == 0:
            x = rng.integers(-2, 1, npg).astype(np.float64)         # ties
        S = x - np.log(np.exp(x).sum())                               # a log-distribution
        if trial % 7 == 0:
            S[rng.integers(0, npg)] = np.nan
        cov = float(rng.choice([0.0, 0.3, 0.5, 0.9, 0.95, 1.0, 1.5]))
        cap = int(rng.integers(1, npg + 2))
        ff = int(rng.integers(0, 3)) if trial % 5 == 0 else 0
        fl = int(rng.integers(0, 3)) if trial % 11 == 0 else 0
        assert coverage_count(S, cov, cap, ff, fl) == _brute_coverage(list(S), cov, cap, ff, fl)


def test_coverage_closed_forms():
    S = np.full(16, math.log(1 / 16))                 # uniform, exact in binary
    assert coverage_count(S, 0.5, 16) == 8
    assert coverage_count(S, 0.51, 16) == 9
    assert coverage_count(S, 1.0, 16) == 16
    assert coverage_count(S, 0.0, 16) == 1             # at least one page
    assert coverage_count(S, 0.95, 4) == 4             # the cap
    dom = np.log(np.array([0.01] * 4 + [0.96]))        # one dominant page
    assert coverage_count(dom, 0.95, 5) == 1
    assert list(select_pages(dom, 1)) == [4]
    # forced pages count with their own mass and are always kept
    assert coverage_count(dom, 0.95, 5, n_force_first=2) == 3
    # NaN pages carry no mass; a prefix that never reaches the coverage keeps every page
    part = np.array([math.log(0.4), math.log(0.4), np.nan])
    assert coverage_count(part, 0.99, 3) == 3
    assert coverage_count(part, 0.8, 3) == 2
    assert coverage_count(part, 0.4, 3) == 1
