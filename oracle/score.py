"""Quad page score (test infrastructure only).

AMASS (amass-kv 0.1.1 project page), section "What is in the box", item 1: a
quadratic, Gaussian-MGF page score built from the per-page summary.  Reading:
the second-order cumulant expansion of the page's log attention mass.  For a
query q, scale tau and the page's keys k_i,

  exact log mass   l(q) = log sum_i exp(tau q.k_i)
  quad score       s(q) = log n + tau q.mu + (tau^2 / 2) sum_{j<=r'} (q.w_j)^2

If the keys were Gaussian with mean mu and covariance sum_j w_j w_j^T, then
log mean_i exp(tau q.k_i) would equal tau q.mu + tau^2 q^T Sigma q / 2, which is
the expression above.  The score is computed from the *stored* summary
(bf16 mu and w, float32 log n), in float64.

Pinned in tests/test_oracle_score.py: n = 1 and identical keys give s = l
exactly; r' >= n - 1 gives the population variance of q.k_i; the two-key
closed form log 2 + 1/2 versus log(e + 1/e); and the large-n Gaussian limit.
"""

import numpy as np


def page_score(q, mu, w, log_n, tau):
    """Quad scores.

    q: (G, d) queries of one KV-head group.  mu: (Np, d), w: (Np, r', d),
    log_n: (Np,).  Returns s_hat (G, Np) float64.
    """
    q = np.asarray(q, dtype=np.float64)
    mu = np.asarray(mu, dtype=np.float64)
    w = np.asarray(w, dtype=np.float64)
    log_n = np.asarray(log_n, dtype=np.float64)
    lin = q @ mu.T                                    # (G, Np)
    proj = np.einsum("gd,prd->gpr", q, w)             # (G, Np, r')
    quad = np.sum(proj * proj, axis=-1)               # (G, Np)
    return log_n[None, :] + tau * lin + 0.5 * tau * tau * quad


def exact_page_logmass(q, keys, tau):
    """l = log sum_i exp(tau q.k_i) for one page; q (G, d), keys (n, d) -> (G,)."""
    z = tau * (np.asarray(q, dtype=np.float64) @ np.asarray(keys, dtype=np.float64).T)
    m = z.max(axis=1, keepdims=True)
    return (m + np.log(np.exp(z - m).sum(axis=1, keepdims=True)))[:, 0]
