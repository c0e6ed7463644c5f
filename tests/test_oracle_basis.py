"""Pins for the shared-basis quad summary and score (CPU only).

The basis against an SVD of the centred keys (a different LAPACK routine);
the page variances by brute-force loops; equality with the per-page quad score
on pages whose centred keys have uncorrelated coordinates along the basis; the
full-rank identity with q^T C q; n = 1 (exact log mass); the hand-worked
two-key page of tests/golden/two_key_page.json; a brute-force score; and
invariance under one rotation applied to keys, basis and queries.
"""

import json
import math
import os

import numpy as np

from oracle.basis import (row_basis, row_covariance, store_basis, basis_page_stats,
                          store_basis_summary, page_score_basis)
from oracle.summary import summarize_page
from oracle.score import page_score, exact_page_logmass

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_basis_matches_svd_subspace_and_is_orthonormal():
    rng = np.random.default_rng(3)
    d, L, r = 24, 400, 4
    # distinct leading variances so the top-r subspace is well separated
    scales = np.concatenate([[5.0, 4.0, 3.0, 2.5], np.full(d - 4, 0.5)])
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    keys = (rng.standard_normal((L, d)) * scales) @ Q.T + rng.standard_normal(d)
    U = row_basis(keys, r)
    np.testing.assert_allclose(U @ U.T, np.eye(r), atol=1e-12)
    Xc = keys - keys.mean(axis=0)
    _, sv, Vt = np.linalg.svd(Xc, full_matrices=False)
    P_svd = Vt[:r].T @ Vt[:r]
    np.testing.assert_allclose(U.T @ U, P_svd, atol=1e-10)
    C = row_covariance(keys)
    np.testing.assert_allclose(np.einsum("rd,de,re->r", U, C, U), sv[:r] ** 2 / L, rtol=1e-10)
    # the covariance itself, by loops on a corner
    m = [sum(keys[t, e] for t in range(L)) / L for e in range(3)]
    for a in range(3):
        for b in range(3):
            ref = sum((keys[t, a] - m[a]) * (keys[t, b] - m[b]) for t in range(L)) / L
            assert abs(C[a, b] - ref) < 1e-12
    # the sign rule makes the output unique
    for j in range(r):
        assert U[j, np.argmax(np.abs(U[j]))] > 0


def test_page_variances_by_loops():
    rng = np.random.default_rng(4)
    n, d, r = 7, 6, 3
    keys = rng.standard_normal((n, d)) * 2 + 1
    U = store_basis(row_basis(rng.standard_normal((50, d)), r))
    mu, lam, log_n = basis_page_stats(keys, U)
    for e in range(d):
        assert abs(mu[e] - sum(keys[i, e] for i in range(n)) / n) < 1e-14
    for j in range(r):
        ref = 0.0
        for i in range(n):
            p = sum(U[j, e] * (keys[i, e] - mu[e]) for e in range(d))
            ref += p * p
        assert abs(lam[j] - ref / n) < 1e-12
    assert log_n == math.log(n)


def test_equals_per_page_score_for_uncorrelated_coordinates():
    # centred keys = a_1 u_1 + a_2 u_2 with Hadamard (orthogonal) coordinate
    # columns of distinct scale: the page's own eigenvectors are u_1, u_2
    rng = np.random.default_rng(5)
    d = 8
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    U = Q[:, :2].T
    mean = rng.standard_normal(d)
    a1 = np.array([1, -1, 1, -1]) * 1.5
    a2 = np.array([1, 1, -1, -1]) * 0.7
    keys = mean + a1[:, None] * U[0] + a2[:, None] * U[1]
    q = rng.standard_normal((3, d))
    tau = 0.4
    mu, lam, log_n = basis_page_stats(keys, U)
    s_basis = page_score_basis(q, mu[None], lam[None], U, np.array([log_n]), tau)[:, 0]
    mu_p, w_p, _, log_n_p = summarize_page(keys, 2)
    s_page = page_score(q, mu_p[None], w_p[None], np.array([log_n_p]), tau)[:, 0]
    np.testing.assert_allclose(s_basis, s_page, rtol=0, atol=1e-12)


def test_full_rank_own_eigenbasis_gives_the_full_quadratic_form():
    rng = np.random.default_rng(6)
    n, d = 9, 5
    keys = rng.standard_normal((n, d))
    C = np.cov(keys.T, bias=True)
    lam_c, vecs = np.linalg.eigh(C)
    U = vecs.T                                   # all d directions
    q = rng.standard_normal((2, d))
    tau = 0.3
    mu, lam, log_n = basis_page_stats(keys, U)
    s = page_score_basis(q, mu[None], lam[None], U, np.array([log_n]), tau)[:, 0]
    ref = math.log(n) + tau * q @ keys.mean(axis=0) + 0.5 * tau * tau * np.einsum("gd,de,ge->g", q, C, q)
    np.testing.assert_allclose(s, ref, rtol=0, atol=1e-12)


def test_single_key_is_exact_log_mass():
    rng = np.random.default_rng(7)
    d = 16
    k = rng.standard_normal((1, d))
    U = store_basis(row_basis(rng.standard_normal((30, d)), 4))
    q = rng.standard_normal((4, d))
    mu, lam, log_n = basis_page_stats(k, U)
    assert np.all(lam == 0)
    s = page_score_basis(q, mu[None], lam[None], U, np.array([log_n]), 0.25)[:, 0]
    np.testing.assert_allclose(s, exact_page_logmass(q, k, 0.25), rtol=0, atol=1e-13)


def test_two_key_worked_page():
    g = json.load(open(os.path.join(GOLDEN, "two_key_page.json")))
    keys = np.array(g["keys"])
    U = row_basis(keys, g["rank"])               # the two keys span (1, 0)
    np.testing.assert_allclose(np.abs(U), np.array(g["w_abs"]), atol=0)
    mu, lam, log_n = basis_page_stats(keys, U)
    np.testing.assert_allclose(lam, g["lambda"], atol=0)
    s = page_score_basis(np.array(g["q"]), mu[None], lam[None], U, np.array([log_n]), g["tau"])[0, 0]
    assert abs(s - g["quad_score"]) < 1e-15


def test_brute_force_score_on_stored_values():
    rng = np.random.default_rng(8)
    G, Np, d, r = 3, 5, 6, 2
    keys = [rng.standard_normal((rng.integers(1, 6), d)) for _ in range(Np)]
    U = store_basis(row_basis(np.concatenate(keys), r))
    stored = [store_basis_summary(*basis_page_stats(k, U)) for k in keys]
    mu = np.array([s[0] for s in stored])
    lam = np.array([s[1] for s in stored])
    log_n = np.array([s[2] for s in stored])
    q = rng.standard_normal((G, d))
    tau = 0.5
    s = page_score_basis(q, mu, lam, U, log_n, tau)
    for h in range(G):
        for p in range(Np):
            lin = sum(q[h, e] * mu[p, e] for e in range(d))
            quad = 0.0
            for j in range(r):
                c = sum(q[h, e] * U[j, e] for e in range(d))
                quad += lam[p, j] * c * c
            assert abs(s[h, p] - (log_n[p] + tau * lin + 0.5 * tau * tau * quad)) < 1e-12
    # stored forms: bf16 mean, float32 variances and log n
    assert all(np.float32(v) == v for v in lam.ravel())
    assert all(np.float32(v) == v for v in log_n)


def test_invariant_under_a_common_rotation():
    rng = np.random.default_rng(9)
    d, r = 10, 3
    keys = rng.standard_normal((12, d)) * np.linspace(3, 0.5, d)
    Q, _ = np.linalg.qr(rng.standard_normal((d, d)))
    q = rng.standard_normal((2, d))
    U = row_basis(keys, r)
    mu, lam, log_n = basis_page_stats(keys, U)
    s1 = page_score_basis(q, mu[None], lam[None], U, np.array([log_n]), 0.3)
    Ur = row_basis(keys @ Q.T, r)
    mu2, lam2, _ = basis_page_stats(keys @ Q.T, Ur)
    s2 = page_score_basis(q @ Q.T, mu2[None], lam2[None], Ur, np.array([log_n]), 0.3)
    np.testing.assert_allclose(s1, s2, rtol=0, atol=1e-10)
