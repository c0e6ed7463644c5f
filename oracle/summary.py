"""Per-page key summary for the quad page score (test infrastructure only).

AMASS (amass-kv 0.1.1 project page), section "What is in the box", item 1: the
quad selector scores pages from a tiny per-page summary that drops the per-key
coordinates and keeps r' eigen-quantities of the page.  The page gives no
formula; the reading taken here (fixed by the method's name, a quadratic
Gaussian moment-generating-function score) is: summarize the n valid keys of a
page by their mean and the top-r' eigenpairs of their population covariance.

Definition, per (page, KV head), over the n valid keys k_1..k_n (rows of X):
  mu     = (1/n) sum_i k_i
  Xc     = X - mu                      (centred keys, n x d)
  Gram   = Xc Xc^T / n                 (n x n; same nonzero spectrum as the
                                        population covariance Xc^T Xc / n)
  (lam_j, v_j) = eigenpairs of Gram, lam descending, negatives clamped to 0
  w_j    = Xc^T v_j / sqrt(n)          (= sqrt(lam_j) u_j, u_j the unit
                                        covariance eigenvector)
  w_j    = 0 when j > n-1 (1-based) or lam_j <= 1e-6 * lam_1
Stored form: bf16(mu), bf16(w_j) (round to nearest even from float64) and
float32(log n).  Directions are stored per page (not a shared basis).

The eigen-decomposition uses numpy.linalg.eigh (LAPACK), a library primitive.
Pinned in tests/test_oracle_summary.py: mean and Gram by brute force, the
eigen residual, agreement of the Gram spectrum with eigh of the d x d
covariance, |w_j|^2 = lam_j, orthogonality, and exact reconstruction of the
covariance when r' >= n - 1.
"""

import math

import numpy as np

from .rounding import round_bf16, as_float32

REL_EIG_FLOOR = 1e-6


def summarize_page(keys, rank):
    """Unrounded summary of one page.

    keys: (n, d) array of the page's valid keys (n >= 1).
    Returns (mu[d], w[rank, d], lam[rank], log_n) in float64.
    """
    X = np.asarray(keys, dtype=np.float64)
    n, d = X.shape
    if n < 1:
        raise ValueError("a page summary needs at least one key")
    # exact column sums rounded once (math.fsum), then divided by n: a page of
    # identical keys has mu equal to that key and no spread at all
    mu = np.array([math.fsum(X[:, e]) for e in range(d)]) / n
    Xc = X - mu
    gram = (Xc @ Xc.T) / n
    lam_all, vecs = np.linalg.eigh(gram)          # ascending
    order = np.argsort(-lam_all, kind="stable")   # descending
    lam_all = np.maximum(lam_all[order], 0.0)
    vecs = vecs[:, order]
    lam1 = lam_all[0]
    w = np.zeros((rank, d), dtype=np.float64)
    lam = np.zeros(rank, dtype=np.float64)
    for j in range(rank):                         # j is 0-based; the rule uses j+1
        if j + 1 > n - 1:
            continue
        if lam_all[j] <= REL_EIG_FLOOR * lam1:
            continue
        lam[j] = lam_all[j]
        w[j] = Xc.T @ vecs[:, j] / np.sqrt(n)
    return mu, w, lam, np.log(n)


def store_summary(mu, w, log_n):
    """Stored form: bf16 mean and directions (as float64 values), float32 log n."""
    return round_bf16(mu), round_bf16(w), np.float64(as_float32(log_n))


def summarize_and_store(keys, rank):
    """summarize_page followed by store_summary; returns (mu_b, w_b, log_n_f32)."""
    mu, w, _lam, log_n = summarize_page(keys, rank)
    return store_summary(mu, w, log_n)
