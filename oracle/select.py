"""Group aggregation and top-k page selection (test infrastructure only).

AMASS (amass-kv 0.1.1 project page), section "Quickstart" (AmassConfig fields
``budget``, a fixed selected-page fraction, and ``coverage``, per-head coverage
over page masses) and section "Benchmarking" (the top-B stage).  Reading taken
for a grouped-query KV head whose G query heads share one selection:

  L_h  = logsumexp_p s_hat[h, p]                       (per-head normaliser)
  a    = s_hat[h, p] - L_h                             (log mass fraction)
  S_p  = log( (1/G) sum_h exp(a[h, p]) )               (group-mean fraction)

computed stably as M_p + log sum_h exp(a - M_p) - log G with M_p = max_h a.
Selection keeps k pages per (sequence, KV head):
  k = k_fixed (clamped to Np) if k_fixed > 0, else
      min(Np, max(1, ceil(keep * Np))) with keep taken as a float32 value and
      the product formed in float64;
  the first n_force_first and the last n_force_last pages get S = +inf;
  order by (S descending, page index ascending), NaN ranking as -inf;
  take the first k and return them in ascending page order.

Coverage mode (the ``coverage`` field: the smallest set of pages holding a given
share of the attention mass).  S_p is a log-distribution (sum_p exp(S_p) = 1),
so with the same ranking (forced pages first by index, then S descending, page
ascending) k is the shortest prefix whose total mass exp(S) reaches the
coverage; forced pages count with their own mass and are always kept, NaN
pages have mass 0; k is then clamped to [max(1, forced pages), min(k_cap, Np)]
and a prefix that never reaches the coverage keeps every page (up to the cap).

Pinned in tests/test_oracle_select.py: sum_p exp(S_p) = 1; G = 1 reduces to the
order of s_hat; a brute-force full sort on tiny inputs over 10^4 seeds; constant
scores select {0..k-1}; forced pages and NaN ranks; coverage counts against a
brute-force loop and closed forms (uniform masses, one dominant page).
"""

import math

import numpy as np


def group_aggregate(s_hat):
    """S_p from per-head quad scores s_hat (G, Np) -> (Np,), float64."""
    s = np.asarray(s_hat, dtype=np.float64)
    G = s.shape[0]
    with np.errstate(invalid="ignore", over="ignore"):
        m_h = s.max(axis=1, keepdims=True)
        L = m_h + np.log(np.exp(s - m_h).sum(axis=1, keepdims=True))
        a = s - L
        M = a.max(axis=0)
        S = M + np.log(np.exp(a - M[None, :]).sum(axis=0)) - math.log(G)
    return S


def selection_count(num_valid_pages, keep_frac, k_fixed=0):
    """k for one row."""
    npg = int(num_valid_pages)
    if npg <= 0:
        return 0
    if k_fixed > 0:
        return min(npg, int(k_fixed))
    keep = float(np.float32(keep_frac))
    return min(npg, max(1, math.ceil(keep * npg)))


def _forced_mask(npg, n_force_first, n_force_last):
    forced = np.zeros(npg, dtype=bool)
    if n_force_first > 0:
        forced[: min(n_force_first, npg)] = True
    if n_force_last > 0:
        forced[max(0, npg - n_force_last):] = True
    return forced


def coverage_count(S, coverage, k_cap, n_force_first=0, n_force_last=0):
    """k for one row in coverage mode (see the module header); S is (Np,)."""
    S = np.array(S, dtype=np.float64)
    npg = S.shape[0]
    if npg == 0:
        return 0
    forced = _forced_mask(npg, n_force_first, n_force_last)
    with np.errstate(over="ignore"):
        mass = np.where(np.isnan(S), 0.0, np.minimum(np.exp(S), 1.0))
    rank_key = np.where(np.isnan(S), -np.inf, S)
    rank_key[forced] = np.inf
    order = np.lexsort((np.arange(npg), -rank_key))
    cum = np.cumsum(mass[order])
    hit = np.nonzero(cum >= coverage)[0]
    k = int(hit[0]) + 1 if hit.size else npg
    k = max(k, int(forced.sum()), 1)
    return min(k, int(k_cap), npg)


def select_pages(S, k, n_force_first=0, n_force_last=0):
    """Indices of the k selected pages, ascending; S is (Np,) for the valid pages."""
    S = np.array(S, dtype=np.float64)
    npg = S.shape[0]
    S[np.isnan(S)] = -np.inf
    if n_force_first > 0:
        S[: min(n_force_first, npg)] = np.inf
    if n_force_last > 0:
        S[max(0, npg - n_force_last):] = np.inf
    idx = np.arange(npg)
    order = np.lexsort((idx, -S))          # primary: S descending; then index ascending
    return np.sort(order[:k]).astype(np.int64)
