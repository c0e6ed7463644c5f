"""Pins of the oracle's r8 low-rank page score against what the mathematics
fixes: exact page log-mass for keys in the span, one-key pages, a brute-force
loop, rotation invariance, coordinates by brute force, empty pages."""

import math

import numpy as np
import pytest

import oracle


def _basis(rng, r, d):
    Q, _ = np.linalg.qr(rng.standard_normal((d, r)))
    return Q.T                                                   # (r, d) orthonormal rows


@pytest.mark.parametrize("seed", range(5))
def test_keys_in_span_give_exact_logmass(seed):
    rng = np.random.default_rng(seed)
    d, r, P, L = 64, 8, 16, 16 * 5 + 3
    U = _basis(rng, r, d)
    m = oracle.round_bf16(rng.standard_normal(d))
    c = oracle.round_bf16(rng.standard_normal((L, r)) * 2)
    keys = m + c @ U
    C = oracle.key_coords(keys, U, m)
    np.testing.assert_array_equal(C, c)                          # coordinates recovered exactly
    q = rng.standard_normal((4, d))
    tau = 1 / math.sqrt(d)
    s = oracle.page_score_lowrank(q, C, m, U, L, P, tau)
    for p in range(s.shape[1]):
        ref = oracle.exact_page_logmass(q, keys[p * P: min((p + 1) * P, L)], tau)
        np.testing.assert_allclose(s[:, p], ref, rtol=0, atol=1e-11)


def test_one_key_page_and_brute_force():
    rng = np.random.default_rng(3)
    d, r, P, L = 32, 8, 4, 4 * 6 + 1
    U = _basis(rng, r, d)
    m = rng.standard_normal(d)
    C = oracle.round_bf16(rng.standard_normal((L, r)))
    q = rng.standard_normal((3, d))
    tau = 0.3
    s = oracle.page_score_lowrank(q, C, m, U, L, P, tau)
    last = L // P                                                # the one-key last page
    kh = m + C[L - 1] @ U
    np.testing.assert_allclose(s[:, last], tau * (q @ kh), rtol=1e-13, atol=1e-13)
    for h in range(q.shape[0]):
        for p in range(s.shape[1]):
            acc = 0.0
            for t in range(p * P, min((p + 1) * P, L)):
                z = tau * (sum(q[h, e] * m[e] for e in range(d)) +
                           sum(sum(q[h, e] * U[j, e] for e in range(d)) * C[t, j] for j in range(r)))
                acc += math.exp(z)
            assert abs(s[h, p] - math.log(acc)) <= 1e-11 * max(1.0, abs(math.log(acc)))


def test_rotation_invariance_and_empty_pages():
    rng = np.random.default_rng(4)
    d, r, P, L = 48, 8, 16, 16 * 3
    U = _basis(rng, r, d)
    m = rng.standard_normal(d)
    C = oracle.round_bf16(rng.standard_normal((L, r)))
    q = rng.standard_normal((2, d))
    R, _ = np.linalg.qr(rng.standard_normal((d, d)))
    s0 = oracle.page_score_lowrank(q, C, m, U, L, P, 0.2)
    s1 = oracle.page_score_lowrank(q @ R, C, m @ R, U @ R, L, P, 0.2)
    np.testing.assert_allclose(s0, s1, rtol=0, atol=1e-11)
    assert oracle.page_score_lowrank(q, C, m, U, 0, P, 0.2).shape == (2, 0)
    assert oracle.page_score_lowrank(q, C, m, U, 17, P, 0.2).shape == (2, 2)


def test_row_lowrank_pieces():
    rng = np.random.default_rng(6)
    keys = oracle.round_bf16(rng.standard_normal((100, 32)) + 0.5)
    U, m, C = oracle.row_lowrank(keys, 90, rank=8)
    np.testing.assert_array_equal(U, oracle.store_basis(oracle.row_basis(keys[:90], 8)))
    mean = np.array([sum(keys[t, e] for t in range(90)) / 90 for e in range(32)])
    np.testing.assert_allclose(m, mean, rtol=2 ** -23, atol=0)
    assert C.shape == (90, 8)
    for t in (0, 45, 89):
        for j in range(8):
            v = sum(U[j, e] * (keys[t, e] - m[e]) for e in range(32))
            assert C[t, j] == oracle.round_bf16(np.array([v]))[0]
