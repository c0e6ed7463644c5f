"""Pins for the quad page score (CPU only).

Closed forms of the second-cumulant expansion: pages whose keys have no spread,
the exact population variance when the rank covers the page, the hand-worked
two-key page in tests/golden/two_key_page.json, and the Gaussian limit in which
the score equals the page's log mass.
"""

import json
import os

import numpy as np

from oracle.summary import summarize_page, summarize_and_store
from oracle.score import page_score, exact_page_logmass

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _score_unrounded(q, keys, rank, tau):
    mu, w, _, log_n = summarize_page(keys, rank)
    return page_score(q, mu[None], w[None], np.array([log_n]), tau)[:, 0]


def test_single_key_and_identical_keys_are_exact():
    rng = np.random.default_rng(0)
    q = rng.standard_normal((4, 64))
    tau = 1 / 8
    k1 = rng.standard_normal((1, 64))
    np.testing.assert_allclose(_score_unrounded(q, k1, 2, tau), exact_page_logmass(q, k1, tau),
                               rtol=0, atol=1e-13)
    same = np.tile(rng.standard_normal(64), (16, 1))
    np.testing.assert_allclose(_score_unrounded(q, same, 2, tau), exact_page_logmass(q, same, tau),
                               rtol=0, atol=1e-13)


def test_full_rank_gives_population_variance():
    rng = np.random.default_rng(1)
    for n in [2, 3, 5]:
        keys = rng.standard_normal((n, 32))
        q = rng.standard_normal((3, 32))
        tau = 0.3
        s = _score_unrounded(q, keys, rank=n - 1, tau=tau)
        z = q @ keys.T                                    # (G, n)
        var = ((z - z.mean(1, keepdims=True)) ** 2).mean(1)
        expect = np.log(n) + tau * z.mean(1) + 0.5 * tau * tau * var
        np.testing.assert_allclose(s, expect, rtol=0, atol=1e-12)


def test_two_key_worked_example():
    g = json.load(open(os.path.join(GOLDEN, "two_key_page.json")))
    keys = np.array(g["keys"])
    q = np.array(g["q"])
    mu, w, lam, log_n = summarize_page(keys, g["rank"])
    np.testing.assert_allclose(mu, g["mu"], atol=1e-15)
    np.testing.assert_allclose(lam, g["lambda"], atol=1e-14)
    np.testing.assert_allclose(np.abs(w), g["w_abs"], atol=1e-14)
    # stored form: bf16 mu/w are exact here, log n is float32
    mu_b, w_b, ln32 = summarize_and_store(keys, g["rank"])
    s = page_score(q, mu_b[None], w_b[None], np.array([ln32]), g["tau"])[0, 0]
    assert abs(s - g["quad_score"]) <= 1e-7
    assert abs(exact_page_logmass(q, keys, g["tau"])[0] - g["exact_logmass"]) <= 1e-14


def test_gaussian_limit_equals_log_mass():
    # keys drawn from a rank-2 Gaussian: log mean exp(tau q.k) -> tau q.mu + tau^2 q^T C q / 2
    rng = np.random.default_rng(2)
    d, n = 8, 200000
    mu0 = rng.standard_normal(d) * 0.3
    A = rng.standard_normal((d, 2)) * 0.4
    keys = mu0 + rng.standard_normal((n, 2)) @ A.T
    q = rng.standard_normal((2, d))
    tau = 0.5
    # summary of the sample, taken from its d x d covariance (the Gram route of
    # the oracle's builder is quadratic in n and is pinned separately)
    mu = keys.mean(0)
    cov = (keys - mu).T @ (keys - mu) / n
    lam, U = np.linalg.eigh(cov)
    w = (U[:, ::-1][:, :2] * np.sqrt(np.maximum(lam[::-1][:2], 0))).T
    s = page_score(q, mu[None], w[None], np.array([np.log(n)]), tau)[:, 0]
    l = exact_page_logmass(q, keys, tau)
    assert np.all(np.abs(s - l) < 1e-2), (s, l)
    # a dropped or doubled quadratic term would miss by far more
    assert np.all(np.abs((s - l)) < 0.1 * np.abs(0.5 * tau * tau * ((q @ A) ** 2).sum(1)))


def test_vectorised_over_pages_and_heads():
    rng = np.random.default_rng(3)
    G, Np, r, d = 4, 6, 2, 16
    mu = rng.standard_normal((Np, d))
    w = rng.standard_normal((Np, r, d))
    ln = rng.standard_normal(Np)
    q = rng.standard_normal((G, d))
    s = page_score(q, mu, w, ln, 0.25)
    for h in range(G):
        for p in range(Np):
            ref = ln[p] + 0.25 * sum(q[h, e] * mu[p, e] for e in range(d))
            ref += 0.5 * 0.0625 * sum(sum(q[h, e] * w[p, j, e] for e in range(d)) ** 2 for j in range(r))
            assert abs(s[h, p] - ref) <= 1e-12
