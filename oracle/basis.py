"""Shared-basis quad summary (test infrastructure only).

AMASS (amass-kv 0.1.1 project page), section "What is in the box", item 1: the
quad summary drops the per-key coordinates and keeps only r' eigenvalues per
page.  Read here with directions shared by every page of a (sequence, KV
head) row: r' directions are computed once per row, as a principal-component
basis of the row's keys, and each page keeps its mean and the variances of
its keys along those directions.  The per-page form in ``oracle.summary``
keeps each page's own directions instead; both feed the same quadratic
Gaussian-MGF score.

Per row, over the keys k_t of all its valid tokens (t < L):
  m        = (1/L) sum_t k_t
  C        = (1/L) sum_t (k_t - m)(k_t - m)^T          population covariance
  u_1..u_r = unit eigenvectors of C for its r' largest eigenvalues
             (numpy.linalg.eigh, a library primitive), descending
  stored   : float32(u_j)  (round to nearest even from float64)
Per page, over its n valid keys, with the stored basis:
  mu       = (1/n) sum_i k_i                           stored bfloat16
  lam_j    = (1/n) sum_i (u_j . (k_i - mu))^2          stored float32 (exact mu)
  log n                                                stored float32
Score of a query q with scale tau, from the stored values, in float64:
  s = log n + tau q.mu + (tau^2 / 2) sum_j lam_j (q.u_j)^2
This is the quad score with the page covariance replaced by its diagonal in
the shared basis.  It equals the per-page form whenever the page's centred
keys lie in span(u) with coordinates that are uncorrelated along the u_j, and
with r' = d and u the page's own eigenbasis it is the full quadratic form
q^T C_page q.

Pinned in tests/test_oracle_basis.py: the basis against an SVD of the centred
keys (a different LAPACK routine) and orthonormality; lam by brute-force loops;
equality with the per-page score on pages with uncorrelated coordinates along
the basis; the full-rank identity; n = 1 (exact page log-mass); the two-key
worked page; a brute-force score; invariance under a common rotation.
"""

import math

import numpy as np

from .rounding import round_bf16, as_float32


def row_basis(keys, rank):
    """Top-`rank` unit eigenvectors of the population covariance of `keys`.

    keys: (L, d) keys of every valid token of the row (L >= 1).
    Returns U (rank, d) float64, rows in descending eigenvalue order.  Each
    row's sign is fixed so that its largest-magnitude entry is positive (the
    score depends on (q.u)^2 only; the sign just makes the output unique).
    """
    X = np.asarray(keys, dtype=np.float64)
    L, d = X.shape
    if L < 1:
        raise ValueError("a basis needs at least one key")
    m = np.array([math.fsum(X[:, e]) for e in range(d)]) / L
    Xc = X - m
    C = (Xc.T @ Xc) / L
    lam, vecs = np.linalg.eigh(C)                 # ascending
    order = np.argsort(-lam, kind="stable")[:rank]
    U = vecs[:, order].T.copy()
    for j in range(U.shape[0]):
        if U[j, np.argmax(np.abs(U[j]))] < 0:
            U[j] = -U[j]
    return U


def row_covariance(keys):
    """The row's population covariance C (d, d), float64 (for invariants)."""
    X = np.asarray(keys, dtype=np.float64)
    m = np.array([math.fsum(X[:, e]) for e in range(X.shape[1])]) / X.shape[0]
    Xc = X - m
    return (Xc.T @ Xc) / X.shape[0]


def store_basis(U):
    """Stored basis: float32 values (as float64)."""
    return as_float32(U).astype(np.float64)


def basis_page_stats(keys, U):
    """Mean, variances along the basis, and log n of one page.

    keys: (n, d) valid keys (n >= 1); U: (r', d) basis as stored.
    Returns (mu[d], lam[r'], log_n) in float64, lam about the exact mean.
    """
    X = np.asarray(keys, dtype=np.float64)
    n, d = X.shape
    if n < 1:
        raise ValueError("a page summary needs at least one key")
    mu = np.array([math.fsum(X[:, e]) for e in range(d)]) / n
    proj = (X - mu) @ np.asarray(U, dtype=np.float64).T      # (n, r')
    lam = (proj * proj).sum(axis=0) / n
    return mu, lam, np.log(n)


def store_basis_summary(mu, lam, log_n):
    """Stored form: bf16 mean, float32 variances and log n (as float64 values)."""
    return (round_bf16(mu), as_float32(lam).astype(np.float64),
            np.float64(as_float32(log_n)))


def page_score_basis(q, mu, lam, U, log_n, tau):
    """Shared-basis quad scores.

    q: (G, d) queries of one KV-head group; mu: (Np, d); lam: (Np, r');
    U: (r', d); log_n: (Np,).  Returns s_hat (G, Np) float64.
    """
    q = np.asarray(q, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    c = q @ np.asarray(U, dtype=np.float64).T                 # (G, r')
    lin = q @ mu.T                                            # (G, Np)
    quad = (c * c) @ lam.T                                    # (G, Np)
    return np.asarray(log_n, dtype=np.float64)[None, :] + tau * lin + 0.5 * tau * tau * quad
