"""Low-rank (r8) page score: per-key coordinates in a shared basis (test
infrastructure only).

AMASS (amass-kv 0.1.1 project page), section "Quickstart" (the `score` field:
`quad` by default, or the `r8` low-rank fallback) and "Headline results" (r8
keeps per-key low-rank state, 15.6 % of the KV cache against the quad
summary's 4.7 %; quad "drops the per-key coordinates" that r8 keeps).  The
page gives no formula; the reading implemented here keeps, for every key, its
coordinates in the row's shared principal basis and scores a page by the
exact log-mass of its keys under that rank-r approximation:

Per (sequence, KV head) row, over the keys k_t of all valid tokens t < L:
  m          = (1/L) sum_t k_t                           stored float32
  u_1..u_r   = the row basis of oracle.basis (r = 8)      stored float32
Per key:
  c_tj       = u_j . (k_t - m)  (exact stored m and u)   stored bfloat16
Score of query q with scale tau, per page p over its n valid tokens, from
the stored values, in float64:
  s_p = tau q.m + log sum_{t in p} exp(tau sum_j (q.u_j) c_tj)
      = log sum_{t in p} exp(tau q . k^_t),   k^_t = m + sum_j c_tj u_j
and -inf for a page with no valid token.

Pinned in tests/test_oracle_lowrank.py: keys that lie in m + span(u) with
coordinates exact in bfloat16 give the exact page log-mass (a different
function, oracle.exact_page_logmass); one-key pages give tau q.k^; a
brute-force loop; invariance under a common rotation of keys, basis and
query; coordinates by brute-force dot products; empty pages.
"""

import math

import numpy as np

from .rounding import round_bf16, as_float32
from .basis import row_basis, store_basis


def row_mean(keys):
    """Mean of the row's valid keys, float64 (exact fsum per element)."""
    X = np.asarray(keys, dtype=np.float64)
    return np.array([math.fsum(X[:, e]) for e in range(X.shape[1])]) / X.shape[0]


def store_mean(m):
    return as_float32(m).astype(np.float64)


def key_coords(keys, U, m):
    """Stored coordinates (n, r) of keys (n, d) in the stored basis U (r, d)
    about the stored mean m: bfloat16 values of u_j . (k - m), as float64."""
    X = np.asarray(keys, dtype=np.float64) - np.asarray(m, dtype=np.float64)
    return round_bf16(X @ np.asarray(U, dtype=np.float64).T)


def row_lowrank(keys, seq_len, rank=8):
    """(U, m, coords) of a row: stored basis, stored mean, stored coordinates
    of every valid key (seq_len, r)."""
    K = np.asarray(keys, dtype=np.float64)[:seq_len]
    U = store_basis(row_basis(K, rank))
    m = store_mean(row_mean(K))
    return U, m, key_coords(K, U, m)


def page_score_lowrank(q, coords, m, U, seq_len, page_size, tau):
    """Scores (G, Np) of every page of a row.

    q: (G, d) query heads; coords: (>= seq_len, r) stored coordinates; m (d,)
    and U (r, d) stored mean and basis."""
    q = np.asarray(q, dtype=np.float64)
    C = np.asarray(coords, dtype=np.float64)[:seq_len]
    qm = tau * (q @ np.asarray(m, dtype=np.float64))                 # (G,)
    qu = q @ np.asarray(U, dtype=np.float64).T                       # (G, r)
    z = tau * (qu @ C.T)                                            # (G, seq_len)
    npg = -(-seq_len // page_size) if seq_len > 0 else 0
    out = np.full((q.shape[0], npg), -np.inf)
    for p in range(npg):
        zz = z[:, p * page_size: min((p + 1) * page_size, seq_len)]
        mx = zz.max(axis=1, keepdims=True)
        out[:, p] = qm + mx[:, 0] + np.log(np.exp(zz - mx).sum(axis=1))
    return out
