"""Tier demotion along the compression cascade (test infrastructure only).

ARGUS (argus_cache 0.1.7.1 project page): section "The One-Minute Explanation"
(hot memory stays in 16-bit for critical, recent and highly attended tokens;
cold memory is compressed progressively from FP8 down to 1-bit), section
"Visual Architecture" (the cascade FP16 -> FP8 -> INT8 -> INT4 -> INT2 ->
1-bit), the telemetry's cascade counts (pages pass through every tier in
turn) and the configuration (max_active_pages and max_fp8_pages as per-tier
page budgets, sink tokens kept in 16-bit).  The page gives no rule beyond
these; the reading implemented here:

  levels  0 native, 1 FP8, 2 int8, 3 int4, 4 int2, 5 1-bit
          (tier ids 0, 5, 1, 2, 3, 4; level 5 has no budget)
  per sequence, over its valid pages p < Np:
    importance  i_p = max over the sequence's KV heads of S[g, p] (the
                group-mean page mass the step's selection ranked by; NaN
                counts as -inf);
    rank        forced pages (the first n_force_first and the last
                n_force_last: sinks and the newest page) first, by index;
                then i descending, page index ascending;
    desired     d_p = the smallest level l <= 4 with
                rank_p < cap_0 + ... + cap_l, else 5;
    new level   current + 1 if d_p > current, else current: a page is
                never promoted (its 16-bit original is gone) and moves at
                most one step per call, as a cascade.
  A demoted page's K and V are decoded from the current tier and the
  encoder's float32 steps are applied to the decoded values.

Pinned in tests/test_oracle_cascade.py: a hand-worked sequence of calls,
convergence of repeated calls to the budgets, agreement of the desired levels
with top-k selection (pinned on its own) at every cumulative budget, the
never-promote / one-step invariants, and the chained codec's consistency and
per-step error bounds.
"""

import numpy as np

from .codec import TIER_NATIVE, TIER_FP8, TIER_I8, TIER_I4, TIER_I2, TIER_B1, encode_vector

TIER_OF_LEVEL = (TIER_NATIVE, TIER_FP8, TIER_I8, TIER_I4, TIER_I2, TIER_B1)
LEVEL_OF_TIER = {t: l for l, t in enumerate(TIER_OF_LEVEL)}
N_BUDGETED = 5


def page_importance(S_heads):
    """(Hkv, Np) group-mean page scores -> (Np,) importance, NaN as -inf."""
    S = np.array(S_heads, dtype=np.float64)
    S[np.isnan(S)] = -np.inf
    return S.max(axis=0)


def rank_pages(importance, n_force_first=0, n_force_last=0):
    """Rank of every page (0 = most important) under the ordering above."""
    imp = np.array(importance, dtype=np.float64)
    npg = imp.shape[0]
    key = imp.copy()
    if n_force_first > 0:
        key[: min(n_force_first, npg)] = np.inf
    if n_force_last > 0:
        key[max(0, npg - n_force_last):] = np.inf
    order = np.lexsort((np.arange(npg), -key))
    rank = np.empty(npg, dtype=np.int64)
    rank[order] = np.arange(npg)
    return rank


def desired_levels(rank, caps):
    """Level each page would hold if demotion were immediate."""
    bounds = np.cumsum(np.asarray(caps, dtype=np.int64)[:N_BUDGETED])
    return np.searchsorted(bounds, np.asarray(rank), side="right")


def plan_row(importance, tiers, caps, n_force_first=0, n_force_last=0):
    """New tier of every valid page of one sequence; tiers are tier ids."""
    level = np.array([LEVEL_OF_TIER[int(t)] for t in tiers], dtype=np.int64)
    d = desired_levels(rank_pages(importance, n_force_first, n_force_last), caps)
    new_level = level + (d > level)
    return np.array([TIER_OF_LEVEL[l] for l in new_level], dtype=np.int64)


def retier_vectors(x, old_tier, new_tier, d):
    """Token vectors held in old_tier (x: their decoded float32 values, which
    for a native page are its 16-bit values) re-encoded into new_tier:
    returns (packed bytes, scale_zero) of the encoder applied to x."""
    assert new_tier != TIER_NATIVE and LEVEL_OF_TIER[new_tier] > LEVEL_OF_TIER[old_tier]
    return encode_vector(np.asarray(x, dtype=np.float32), new_tier)

