"""Pins for the per-page summary (CPU only).

Checked against brute-force sums, an SVD of the centred keys (a different
LAPACK routine from the oracle's Gram eigh), and the algebraic identities the
definition implies.
"""

import numpy as np
import scipy.linalg

from oracle.summary import summarize_page, store_summary, summarize_and_store
from oracle.rounding import round_bf16


def _rand_page(seed, n, d, scale=1.0):
    return np.random.default_rng(seed).standard_normal((n, d)) * scale


def test_mean_and_gram_brute_force():
    X = _rand_page(0, 5, 6)
    n, d = X.shape
    mu_bf = [sum(X[i][e] for i in range(n)) / n for e in range(d)]
    mu, w, lam, log_n = summarize_page(X, rank=4)
    np.testing.assert_allclose(mu, mu_bf, rtol=0, atol=1e-15)
    assert log_n == np.log(5)
    # r' = 4 = n - 1: sum_j w_j w_j^T must be the population covariance, entry by entry
    cov_bf = np.zeros((d, d))
    for i in range(n):
        for a in range(d):
            for b in range(d):
                cov_bf[a, b] += (X[i, a] - mu_bf[a]) * (X[i, b] - mu_bf[b]) / n
    np.testing.assert_allclose(w.T @ w, cov_bf, rtol=0, atol=1e-12)


def test_spectrum_matches_svd_of_centred_keys():
    for seed, (n, d) in enumerate([(16, 128), (32, 128), (16, 64), (7, 64), (3, 8)]):
        X = _rand_page(seed, n, d)
        r = 4
        mu, w, lam, _ = summarize_page(X, r)
        sv = scipy.linalg.svd((X - X.mean(0)) / np.sqrt(n), compute_uv=False)
        ref = sv[:r] ** 2
        for j in range(r):
            if j + 1 > n - 1:
                assert lam[j] == 0.0 and not w[j].any()
            else:
                assert abs(lam[j] - ref[j]) <= 1e-10 * ref[0]
                assert abs(w[j] @ w[j] - ref[j]) <= 1e-10 * ref[0]


def test_eigen_residual_and_orthogonality():
    X = _rand_page(5, 16, 128)
    n = X.shape[0]
    mu, w, lam, _ = summarize_page(X, 4)
    Xc = X - mu
    cov = Xc.T @ Xc / n
    norm = np.linalg.norm(cov)
    for j in range(4):
        u = w[j] / np.linalg.norm(w[j])
        assert np.linalg.norm(cov @ u - lam[j] * u) <= 1e-10 * norm
        for i in range(j):
            assert abs(w[i] @ w[j]) <= 1e-10 * norm
    assert np.all(np.diff(lam) <= 0)


def test_invariant_to_token_order():
    X = _rand_page(7, 16, 128)
    perm = np.random.default_rng(8).permutation(16)
    _, w1, l1, _ = summarize_page(X, 4)
    _, w2, l2, _ = summarize_page(X[perm], 4)
    np.testing.assert_allclose(l1, l2, rtol=1e-12)
    np.testing.assert_allclose(w1.T @ w1, w2.T @ w2, atol=1e-12)


def test_degenerate_pages():
    k = np.random.default_rng(3).standard_normal(64)
    mu, w, lam, log_n = summarize_page(k[None, :], 2)          # n = 1
    np.testing.assert_array_equal(mu, k)
    assert not w.any() and log_n == 0.0
    mu, w, lam, _ = summarize_page(np.tile(k, (16, 1)), 2)     # constant page
    np.testing.assert_allclose(mu, k, atol=1e-15)
    assert not w.any()
    two = np.stack([k, -k])                                     # rank one, n = 2
    mu, w, lam, _ = summarize_page(two, 4)
    assert lam[0] > 0 and not w[1:].any()


def test_relative_eigen_floor():
    rng = np.random.default_rng(9)
    u = rng.standard_normal(32)
    v = rng.standard_normal(32)
    v -= (v @ u) / (u @ u) * u
    coeff = rng.standard_normal((16, 2))
    coeff -= coeff.mean(0)
    # second direction carries variance ~1e-8 of the first: below the 1e-6 floor
    X = coeff[:, :1] * u + 1e-4 * coeff[:, 1:] * v
    _, w, lam, _ = summarize_page(X, 2)
    assert lam[0] > 0 and lam[1] == 0.0 and not w[1].any()


def test_stored_form():
    X = _rand_page(11, 16, 128)
    mu, w, lam, log_n = summarize_page(X, 4)
    mu_b, w_b, ln32 = store_summary(mu, w, log_n)
    np.testing.assert_array_equal(mu_b, round_bf16(mu))
    np.testing.assert_array_equal(w_b, round_bf16(w))
    assert ln32 == np.float64(np.float32(np.log(16)))
    # bf16 keeps 8 significant bits
    nz = mu != 0
    assert np.all(np.abs(mu_b[nz] - mu[nz]) <= np.abs(mu[nz]) * 2.0 ** -8)
    a, b, c = summarize_and_store(X, 4)
    np.testing.assert_array_equal(a, mu_b)
    np.testing.assert_array_equal(b, w_b)
    assert c == ln32
