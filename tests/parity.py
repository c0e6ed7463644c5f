"""Comparison helpers shared by the GPU parity tests (imports the oracle; test-only).

Acceptance rules:
* quad scores: |gpu - oracle| <= 1e-5 * max(1, |oracle|) on the same stored summary;
* selection: pages whose oracle S is within 1e-5 * max(1, |S|, |S_k|) of the
  k-th score S_k are interchangeable; the GPU set must have exactly k pages,
  contain every oracle page above that band and none below it;
* attention: max abs error <= 2e-3 per output element and per lse.
"""

import numpy as np

import oracle
from quantized_kv_cache_summary_amd import workloads as wl

SCORE_REL = 1e-5
BAND_REL = 1e-5
ATTN_ABS = 2e-3


def assert_scores_close(gpu, ref, rel=SCORE_REL, what="scores"):
    gpu = np.asarray(gpu, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    assert gpu.shape == ref.shape
    tol = rel * np.maximum(1.0, np.abs(ref))
    err = np.abs(gpu - ref)
    bad = ~(err <= tol)
    assert not bad.any(), f"{what}: {bad.sum()} of {bad.size} outside tol; worst {np.nanmax(err / tol):.3g}x"
    return float(np.max(err)) if err.size else 0.0


def check_selection(S_ref, k, sel_gpu, rel=BAND_REL, forced=()):
    """Returns the number of in-band pages on which the two sets differ."""
    S = np.array(S_ref, dtype=np.float64)
    S[np.isnan(S)] = -np.inf
    for p in forced:
        S[p] = np.inf
    sel = np.asarray(sel_gpu, dtype=np.int64)
    assert sel.size == k, (sel.size, k)
    assert np.all(np.diff(sel) > 0), "selection not strictly ascending"
    assert sel.min(initial=0) >= 0 and sel.max(initial=-1) < S.size
    if k == 0:
        return 0
    order = np.lexsort((np.arange(S.size), -S))
    Sk = S[order[k - 1]]
    if np.isinf(Sk):
        tol = 0.0
        above = S > Sk
        below = S < Sk
    else:
        tol = rel * np.maximum(1.0, np.maximum(np.abs(np.where(np.isinf(S), 0, S)), abs(Sk)))
        above = S > Sk + tol
        below = S < Sk - tol
    chosen = np.zeros(S.size, bool)
    chosen[sel] = True
    assert np.all(chosen[above]), f"missing pages above the band: {np.nonzero(above & ~chosen)[0][:10]}"
    assert not np.any(chosen[below]), f"pages below the band chosen: {np.nonzero(below & chosen)[0][:10]}"
    ref_sel = oracle.select_pages(S_ref, k, 0, 0) if not forced else None
    if ref_sel is None:
        return 0
    return int(np.setdiff1d(sel, ref_sel).size)


def assert_attn_close(out_gpu, lse_gpu, out_ref, lse_ref, tol=ATTN_ABS):
    out_gpu = np.asarray(out_gpu, np.float64)
    out_ref = np.asarray(out_ref, np.float64)
    assert np.array_equal(np.isnan(out_gpu), np.isnan(out_ref))
    err = np.nanmax(np.abs(out_gpu - out_ref)) if out_ref.size else 0.0
    assert err <= tol, f"out max abs err {err}"
    lg, lr = np.asarray(lse_gpu, np.float64), np.asarray(lse_ref, np.float64)
    inf = np.isinf(lr)
    assert np.array_equal(np.isinf(lg), inf) and np.all(lg[inf] == lr[inf])
    fin = ~inf & ~np.isnan(lr)
    lerr = np.max(np.abs(lg[fin] - lr[fin])) if fin.any() else 0.0
    assert lerr <= tol, f"lse max abs err {lerr}"
    return float(err), float(lerr)


def row_summary_from_records(rec_f64, bt_row, Np, rank, d):
    """Stored summary of a row's logical pages from a per-physical-page record table
    rec_f64 [n_phys, Hkv_slice..., (1+R)*d] already sliced to the KV head."""
    r = rec_f64[bt_row[:Np]].reshape(Np, 1 + rank, d)
    return r[:, 0], r[:, 1:]


def bits_to_f64(bits, dtype="bf16"):
    return wl.bits_to_f32(bits, dtype).astype(np.float64)
