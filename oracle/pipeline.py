"""One decode step for one (sequence, KV head) row (test infrastructure only).

Chains the oracle's steps in the order the AMASS page gives them (amass-kv
0.1.1 project page, sections "AMASS" and "What is in the box"): score every
page from its summary, select the top pages, attend over the selected pages
only.  Packed-tier pages are reconstructed before attention (ARGUS,
argus_cache 0.1.7.1 project page, section "Why It Works: Storage vs.
Computation"); their summaries are built from the original 16-bit keys at
append time, before packing.
"""

import numpy as np

from .paging import num_pages, page_token_counts
from .summary import summarize_and_store
from .score import page_score
from .basis import row_basis, store_basis, basis_page_stats, store_basis_summary, page_score_basis
from .select import group_aggregate, selection_count, select_pages, coverage_count
from .attention import sparse_attention
from .codec import TIER_NATIVE, encode_vector, decode_vector


def build_row_summaries(keys, seq_len, page_size, rank):
    """Stored summaries of every logical page of one row."""
    keys = np.asarray(keys, dtype=np.float64)
    npg = num_pages(seq_len, page_size)
    d = keys.shape[1]
    mu = np.zeros((npg, d))
    w = np.zeros((npg, rank, d))
    log_n = np.zeros(npg)
    for p in range(npg):
        lo = p * page_size
        mu[p], w[p], log_n[p] = summarize_and_store(keys[lo:min(lo + page_size, seq_len)], rank)
    return mu, w, log_n


def build_row_basis_summaries(keys, seq_len, page_size, rank, basis=None):
    """Shared-basis stored summaries of every logical page of one row.

    basis: the stored (r', d) basis to use; by default the row's own
    (row_basis over its seq_len valid keys, stored as float32).
    Returns (U, mu, lam, log_n).
    """
    keys = np.asarray(keys, dtype=np.float64)[:seq_len]
    U = store_basis(row_basis(keys, rank)) if basis is None else np.asarray(basis, dtype=np.float64)
    npg = num_pages(seq_len, page_size)
    d = keys.shape[1]
    mu = np.zeros((npg, d))
    lam = np.zeros((npg, U.shape[0]))
    log_n = np.zeros(npg)
    for p in range(npg):
        lo = p * page_size
        mu[p], lam[p], log_n[p] = store_basis_summary(
            *basis_page_stats(keys[lo:min(lo + page_size, seq_len)], U))
    return U, mu, lam, log_n


def reconstruct_tiers(x, seq_len, page_size, page_tiers, b1_outliers=False):
    """Encode and decode every token vector of the non-native pages (float64 out);
    with b1_outliers the 1-bit pages keep their outlier side-table elements."""
    x = np.array(x, dtype=np.float64)
    if page_tiers is None:
        return x
    d = x.shape[1]
    for p, tier in enumerate(page_tiers):
        if tier == TIER_NATIVE:
            continue
        lo, hi = p * page_size, min((p + 1) * page_size, seq_len)
        enc = encode_vector(x[lo:hi].astype(np.float32), int(tier), outliers=b1_outliers)
        x[lo:hi] = decode_vector(enc[0], enc[1], int(tier), d, outlier=enc[2] if len(enc) > 2 else None)
    return x


def decode_row(q, keys, values, seq_len, page_size, rank, tau, keep_frac=0.0, k_fixed=0,
               n_force_first=0, n_force_last=0, page_tiers=None, summary=None, shared_basis=False,
               basis=None, coverage=None, k_cap=None):
    """Full step for one row.

    q: (G, d); keys, values: (>= seq_len, d) 16-bit values in logical token order.
    summary: optional stored summary to score from -- (mu, w, log_n) per page,
    or (U, mu, lam, log_n) with shared_basis -- built here otherwise (with
    shared_basis, from `basis` if given, else the row's own basis).
    coverage: coverage mode (k from the mass prefix, capped at k_cap) instead of
    keep_frac / k_fixed.
    """
    keys = np.asarray(keys, dtype=np.float64)[:seq_len]
    values = np.asarray(values, dtype=np.float64)[:seq_len]
    npg = num_pages(seq_len, page_size)
    if shared_basis:
        if summary is None:
            summary = build_row_basis_summaries(keys, seq_len, page_size, rank, basis)
        U, mu, w, log_n = summary                # w holds the per-page variances here
        s_hat = page_score_basis(q, mu[:npg], w[:npg], U, log_n[:npg], tau)
    else:
        if summary is None:
            summary = build_row_summaries(keys, seq_len, page_size, rank)
        mu, w, log_n = summary
        s_hat = page_score(q, mu[:npg], w[:npg], log_n[:npg], tau)
    S = group_aggregate(s_hat) if npg else np.zeros(0)
    if coverage is None:
        k = selection_count(npg, keep_frac, k_fixed)
    else:
        k = coverage_count(S, coverage, npg if k_cap is None else k_cap, n_force_first, n_force_last)
    sel = select_pages(S, k, n_force_first, n_force_last) if npg else np.zeros(0, np.int64)
    k_hat = reconstruct_tiers(keys, seq_len, page_size, page_tiers)
    v_hat = reconstruct_tiers(values, seq_len, page_size, page_tiers)
    out, lse = sparse_attention(q, k_hat, v_hat, seq_len, page_size, sel, tau)
    return dict(mu=mu, w=w, log_n=log_n, s_hat=s_hat, S=S, k=k, sel=sel, out=out, lse=lse,
                n_valid=page_token_counts(seq_len, page_size))
