"""GPU parity of every kernel against the oracle, at sizes the oracle finishes in
seconds that still span several tiles and a ragged tail, plus edge cases.

Inputs come from the seeded generator only; the oracle recomputes from the same
inputs and never sees a GPU result except to compare.
"""

import math

import numpy as np
import pytest
import torch

import oracle
from oracle.pipeline import reconstruct_tiers
from parity import (assert_scores_close, check_selection, assert_attn_close, bits_to_f64, ATTN_ABS)
from quantized_kv_cache_summary_amd import workloads as wl

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS
SMALL = {
    "tiny": W["tiny"],
    "llama_small": W["llama8b_32k"].replace(B=2, ctx=16 * 300 + 7),        # 301 pages, 7-token tail
    "qwen_small": W["qwen3b_128k"].replace(B=2, ctx=16 * 400),             # G = 8
    "heavy_small": W["heavy70b_128k"].replace(B=2, Hq=16, Hkv=2, ctx=32 * 150 + 5, v_host=False),  # P = 32
}
# summary builder only: clustered (low-rank) keys, and float16 keys at P = 32
SUMMARY_ONLY = {
    "gmm_small": W["tiers_64k"].replace(B=2, ctx=16 * 120 + 9, keys="gmm", gmm_centers=64, gmm_std=0.5),
    "heavy_f16_small": W["heavy70b_128k"].replace(B=2, Hq=16, Hkv=2, ctx=32 * 60 + 17, v_host=False,
                                                  dtype="f16"),
    # the solver's other group widths: rank 8 (8 lanes per eigenvalue) at page
    # sizes 16 and 32 and rank 1 (one group of 64 lanes); the tiny workload has rank 2
    "r8_p16": W["llama8b_32k"].replace(B=2, Hq=8, Hkv=2, ctx=16 * 90 + 11, rank=8),
    "r8_p32": W["heavy70b_128k"].replace(B=2, Hq=16, Hkv=2, ctx=32 * 45 + 21, v_host=False, rank=8),
    "r1_p16": W["llama8b_32k"].replace(B=2, Hq=8, Hkv=2, ctx=16 * 90 + 5, rank=1),
}


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def hz():
    from quantized_kv_cache_summary_amd import harness
    return harness


def _q_ref(w, b, g, qidx=0):
    return wl.queries(w, 0, b, g, qidx).astype(np.float64)


# ---------------------------------------------------------------- score + select

@pytest.mark.parametrize("name", list(SMALL))
def test_score_and_select_parity(hz, name):
    w = SMALL[name]
    L = w.ctx
    lens = [L, max(1, L - 3 * w.P - 5)] if w.B == 2 else [L]
    announce(f"score/select {name} seq_lens={lens}")
    layer = hz.DeviceLayer(w, summaries="synthetic", seq_lens=lens)
    q = hz.queries_device(w)
    bufs = hz.StepBuffers(w, with_S=True)
    hz.score(layer, q, bufs)
    hz.topk(layer, bufs)
    torch.cuda.synchronize()
    hs = bufs.head_scores.cpu().numpy()
    S_gpu = bufs.page_S.cpu().numpy()
    sel = bufs.sel.cpu().numpy()
    cnt = bufs.sel_count.cpu().numpy()
    rec_bits, n_valid = wl.synthetic_summary(w)
    rec = bits_to_f64(rec_bits)                    # [B, Hkv, Np, 1+R, d], logical page order
    log_n = np.log(n_valid.astype(np.float64)).astype(np.float32).astype(np.float64)
    swaps = 0
    for b in range(w.B):
        Np = oracle.num_pages(lens[b], w.P)
        for g in range(w.Hkv):
            s_ref = oracle.page_score(_q_ref(w, b, g), rec[b, g, :Np, 0], rec[b, g, :Np, 1:], log_n[b, :Np], w.tau)
            assert_scores_close(hs[b, g, :, :Np], s_ref)
            assert np.all(hs[b, g, :, Np:] == -np.inf)
            S_ref = oracle.group_aggregate(s_ref)
            assert_scores_close(S_gpu[b, g, :Np], S_ref, what="S")
            assert abs(np.exp(S_gpu[b, g, :Np].astype(np.float64)).sum() - 1) < 1e-5
            k = oracle.selection_count(Np, w.keep, w.k_fixed)
            assert cnt[b, g] == k
            swaps += check_selection(S_ref, k, sel[b, g, :k])
            assert np.all(sel[b, g, k:] == -1)
    print(f"in-band swaps: {swaps}")


def test_forced_pages_and_fixed_k(hz):
    w = SMALL["llama_small"]
    announce("forced pages / k_fixed")
    layer = hz.DeviceLayer(w, summaries="synthetic")
    q = hz.queries_device(w)
    bufs = hz.StepBuffers(w.replace(k_fixed=20), with_S=True)
    hz.score(layer, q, bufs)
    from quantized_kv_cache_summary_amd import kvsparse as kv
    kv.page_topk(layer.L, bufs.head_scores, bufs.lse_partial, layer.seq_lens, w.Np, 0.0, 20, bufs.sel,
                 bufs.sel_count, n_force_first=2, n_force_last=3, page_S=bufs.page_S)
    torch.cuda.synchronize()
    S = bufs.page_S.cpu().numpy().astype(np.float64)
    sel = bufs.sel.cpu().numpy()
    rec_bits, n_valid = wl.synthetic_summary(w)
    rec = bits_to_f64(rec_bits)
    log_n = np.log(n_valid.astype(np.float64)).astype(np.float32).astype(np.float64)
    for b in range(w.B):
        for g in range(w.Hkv):
            s_ref = oracle.page_score(_q_ref(w, b, g), rec[b, g, :, 0], rec[b, g, :, 1:], log_n[b], w.tau)
            S_ref = oracle.group_aggregate(s_ref)
            forced = [0, 1, w.Np - 3, w.Np - 2, w.Np - 1]
            assert all(np.isinf(S[b, g, p]) for p in forced)
            check_selection(S_ref, 20, sel[b, g, :20], forced=forced)
            assert set(forced) <= set(sel[b, g, :20].tolist())


def _tile_partials(hs, Np, n_tiles, tile=64):
    """(max, sum exp(x - max)) of every 64-page tile and head over the finite
    scores of pages < Np: the per-block partials the score kernel leaves."""
    rows, G, _ = hs.shape
    part = np.zeros((rows, n_tiles, G, 2), np.float32)
    for r in range(rows):
        for t in range(n_tiles):
            for h in range(G):
                x = hs[r, h, t * tile:min((t + 1) * tile, Np[r])].astype(np.float64)
                x = x[np.isfinite(x)]
                if x.size == 0:
                    part[r, t, h] = (-np.inf, 0.0)
                else:
                    m = x.max()
                    part[r, t, h] = (m, np.exp(x - m).sum())
    return part


def _crafted_scores(G, max_pages, rng):
    """Rows that reach every branch of the selector: heavy exact ties, a wide
    range, keys that differ only in the last mantissa bits, mostly -inf, NaN
    scores, all equal, an empty row and a short one."""
    Np = np.array([max_pages, 577, 600, 590, 512, 333, 0, 3])
    hs = np.full((8, G, max_pages), -np.inf, np.float32)
    hs[0, :, :Np[0]] = rng.integers(0, 4, (G, Np[0]))
    hs[1, :, :Np[1]] = rng.standard_normal((G, Np[1])) * 30
    base = np.float32(5.0)
    steps = (np.arange(Np[2]) % 37).astype(np.float32)
    hs[2, :, :Np[2]] = base + steps * np.float32(2.0 ** -20)
    fin = rng.choice(Np[3], 5, replace=False)
    hs[3, :, fin] = rng.standard_normal((5, G))
    hs[4, :, :Np[4]] = rng.standard_normal((G, Np[4]))
    hs[4, 1, rng.choice(Np[4], 40, replace=False)] = np.nan
    hs[5, :, :Np[5]] = 2.5
    hs[7, :, :Np[7]] = rng.standard_normal((G, Np[7]))
    return hs, Np


def _expected_selection(S, Np, k):
    """Top k of float32 scores by (S descending, page ascending), NaN as -inf."""
    x = np.where(np.isnan(S[:Np]), -np.inf, S[:Np]).astype(np.float64)
    order = np.lexsort((np.arange(Np), -x))
    return np.sort(order[:k])


@pytest.mark.parametrize("G,max_pages", [(4, 600), (8, 600), (16, 600), (4, 5000), (16, 5000), (4, 15360)])
def test_selection_branches_exact(G, max_pages):
    """Selection on crafted head scores, checked bit-exactly against an
    exhaustive sort of the kernel's own float32 S (the order is unique given S).
    Rows of 4096 pages or more take the selector's wide-block variant; 15360
    pages is the longest row the selector takes (its keys fill 60 KB of LDS)."""
    from quantized_kv_cache_summary_amd import kvsparse as kv
    announce(f"crafted selection G={G} max_pages={max_pages}")
    rng = np.random.default_rng(17 + G)
    n_tiles = (max_pages + 63) // 64
    L = kv.layout(G, 1, 128, 16, 4, "bf16")
    hs, Np = _crafted_scores(G, max_pages, rng)
    part = _tile_partials(hs, Np, n_tiles)
    seq = torch.tensor(Np * 16 - (Np > 0) * 5, dtype=torch.int32, device="cuda")   # ragged last page
    hs_d = torch.from_numpy(hs).cuda()
    part_d = torch.from_numpy(part).cuda()
    cases = [(0.1, 0, 0, 0), (0.0, 7, 0, 0), (0.0, 5, 6, 4), (0.0, 12, 6, 4), (1.0, 0, 0, 0)]
    for keep, k_fixed, nff, nfl in cases:
        k_max = oracle.selection_count(max_pages, keep, k_fixed)
        sel = torch.full((8, k_max), -7, dtype=torch.int32, device="cuda")
        cnt = torch.zeros(8, dtype=torch.int32, device="cuda")
        S = torch.zeros((8, max_pages), dtype=torch.float32, device="cuda")
        kv.page_topk(L, hs_d, part_d, seq, max_pages, keep, k_fixed, sel, cnt, n_force_first=nff,
                     n_force_last=nfl, page_S=S)
        torch.cuda.synchronize()
        S_h, sel_h, cnt_h = S.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy()
        for r in range(8):
            k = oracle.selection_count(int(Np[r]), keep, k_fixed)
            assert cnt_h[r] == k, (keep, k_fixed, r)
            if Np[r] > 0:
                forced = [p for p in range(Np[r]) if p < nff or p >= Np[r] - nfl]
                assert np.all(np.isposinf(S_h[r, forced]))
            exp = _expected_selection(S_h[r], int(Np[r]), k)
            assert np.array_equal(sel_h[r, :k], exp), (keep, k_fixed, nff, nfl, r)
            assert np.all(sel_h[r, k:] == -1)


def _coverage_bounds(S, Np, cov, cap, nff, nfl, delta):
    """Range of coverage counts for coverages within +-delta (counts are monotone)."""
    lo = oracle.coverage_count(S[:Np], max(0.0, cov - delta), cap, nff, nfl)
    hi = oracle.coverage_count(S[:Np], cov + delta, cap, nff, nfl)
    return lo, hi


@pytest.mark.parametrize("G,max_pages", [(4, 600), (8, 600), (4, 5000), (8, 15360)])
def test_coverage_selection_crafted(G, max_pages):
    """Coverage mode on crafted head scores: k within the counts for coverages
    +-1e-6 around the asked one, computed from the kernel's own float32 S
    (masses are summed in 2^-40 fixed point), and the kept pages are exactly
    the top k of that S."""
    from quantized_kv_cache_summary_amd import kvsparse as kv
    announce(f"coverage selection G={G} max_pages={max_pages}")
    rng = np.random.default_rng(29 + G)
    n_tiles = (max_pages + 63) // 64
    L = kv.layout(G, 1, 128, 16, 4, "bf16")
    hs, Np = _crafted_scores(G, max_pages, rng)
    part = _tile_partials(hs, Np, n_tiles)
    seq = torch.tensor(Np * 16 - (Np > 0) * 5, dtype=torch.int32, device="cuda")
    hs_d = torch.from_numpy(hs).cuda()
    part_d = torch.from_numpy(part).cuda()
    cases = [(0.95, max_pages, 0, 0), (0.5, max_pages, 0, 0), (0.0, max_pages, 0, 0), (1.0, max_pages, 0, 0),
             (1.5, 40, 0, 0), (0.9, 25, 0, 0), (0.95, max_pages, 3, 2), (0.2, max_pages, 6, 0),
             (0.6, max_pages, 0, 5), (0.99, 30, 2, 2)]
    # the kernel's own float32 S of every page, forced ones included: page_S of
    # a call without forced pages (S does not depend on forcing; forced pages
    # count with their own mass and only rank first)
    S_all = torch.zeros((8, max_pages), dtype=torch.float32, device="cuda")
    kv.page_topk_coverage(L, hs_d, part_d, seq, max_pages, 0.5,
                          torch.full((8, max_pages), -7, dtype=torch.int32, device="cuda"),
                          torch.zeros(8, dtype=torch.int32, device="cuda"), page_S=S_all)
    torch.cuda.synchronize()
    S_all = S_all.cpu().numpy().astype(np.float64)
    seen = set()
    for cov, cap, nff, nfl in cases:
        sel = torch.full((8, cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((8,), -7, dtype=torch.int32, device="cuda")
        S = torch.zeros((8, max_pages), dtype=torch.float32, device="cuda")
        kv.page_topk_coverage(L, hs_d, part_d, seq, max_pages, cov, sel, cnt, n_force_first=nff,
                              n_force_last=nfl, page_S=S)
        torch.cuda.synchronize()
        S_h, sel_h, cnt_h = S.cpu().numpy(), sel.cpu().numpy(), cnt.cpu().numpy()
        for r in range(8):
            n = int(Np[r])
            k = int(cnt_h[r])
            if n == 0:
                assert k == 0 and np.all(sel_h[r] == -1)
                continue
            # forced pages hold +inf in page_S; their masses come from the unforced call's S
            Sr = S_h[r].astype(np.float64)
            forced = [p for p in range(n) if p < nff or p >= n - nfl]
            assert np.all(np.isposinf(Sr[forced]))
            assert np.array_equal(np.delete(Sr[:n], forced).view(np.uint64),
                                  np.delete(S_all[r, :n], forced).view(np.uint64))
            lo, hi = _coverage_bounds(S_all[r], n, cov, cap, nff, nfl, 1e-6)
            assert lo <= k <= hi, (cov, cap, nff, nfl, r, k, lo, hi)
            assert max(1, len(forced)) <= k <= min(cap, n)
            seen.add(k)
            exp = _expected_selection(S_h[r], n, k)
            assert np.array_equal(sel_h[r, :k], exp), (cov, r)
            assert np.all(sel_h[r, k:] == -1)
    assert len(seen) > 4


def test_coverage_selection_on_scores(hz):
    """Coverage mode from real scores against the oracle's coverage count on its
    own S, within a 1e-5 mass band, and the band-exact selection."""
    from quantized_kv_cache_summary_amd import kvsparse as kv
    w = SMALL["llama_small"]
    lens = [w.ctx, w.ctx - 3 * w.P - 5]
    announce("coverage selection on llama_small scores")
    layer = hz.DeviceLayer(w, summaries="synthetic", seq_lens=lens)
    q = hz.queries_device(w)
    bufs = hz.StepBuffers(w, with_S=True)
    hz.score(layer, q, bufs)
    rec_bits, n_valid = wl.synthetic_summary(w)
    rec = bits_to_f64(rec_bits)
    log_n = np.log(n_valid.astype(np.float64)).astype(np.float32).astype(np.float64)
    S_ref = {}
    for b in range(w.B):
        Np = oracle.num_pages(lens[b], w.P)
        for g in range(w.Hkv):
            s_ref = oracle.page_score(_q_ref(w, b, g), rec[b, g, :Np, 0], rec[b, g, :Np, 1:], log_n[b, :Np], w.tau)
            S_ref[b, g] = oracle.group_aggregate(s_ref)
    for cov, cap, nff, nfl in ((0.3, w.Np, 0, 0), (0.8, w.Np, 0, 0), (0.95, w.Np, 0, 0), (0.8, w.Np, 3, 2),
                               (0.5, w.Np, 0, 4), (0.95, 100, 2, 0)):
        sel = torch.full((w.B, w.Hkv, cap), -7, dtype=torch.int32, device="cuda")
        cnt = torch.zeros((w.B, w.Hkv), dtype=torch.int32, device="cuda")
        kv.page_topk_coverage(layer.L, bufs.head_scores, bufs.lse_partial, layer.seq_lens, w.Np, cov, sel, cnt,
                              n_force_first=nff, n_force_last=nfl)
        torch.cuda.synchronize()
        sel_h, cnt_h = sel.cpu().numpy(), cnt.cpu().numpy()
        for b in range(w.B):
            Np = oracle.num_pages(lens[b], w.P)
            for g in range(w.Hkv):
                k = int(cnt_h[b, g])
                lo, hi = _coverage_bounds(S_ref[b, g], Np, cov, cap, nff, nfl, 1e-5)
                assert lo <= k <= hi, (cov, cap, nff, nfl, b, g, k, lo, hi)
                forced = [p for p in range(Np) if p < nff or p >= Np - nfl]
                check_selection(S_ref[b, g], k, sel_h[b, g, :k], forced=forced)
                assert np.all(sel_h[b, g, k:] == -1)


# ---------------------------------------------------------------- attention

@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_attention_parity_random_selection(hz, name, splits):
    w = SMALL[name]
    lens = [w.ctx, max(1, w.ctx - 2 * w.P - 3)] if w.B == 2 else [w.ctx]
    announce(f"attention {name} splits={splits} seq_lens={lens}")
    layer = hz.DeviceLayer(w, summaries=None, seq_lens=lens)
    q = hz.queries_device(w)
    k = w.k_of(w.Np)
    sel_np, cnt_np = wl.synthetic_selection(w, k, ragged=True)
    bufs = hz.StepBuffers(w, num_splits=splits)
    hz.attend(layer, q, bufs, sel=torch.from_numpy(sel_np).cuda(), sel_count=torch.from_numpy(cnt_np).cuda())
    torch.cuda.synchronize()
    out = bufs.out.cpu().numpy()
    lse = bufs.lse.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            K = wl.row_keys(w, 0, b, g)
            V = wl.row_values(w, 0, b, g)
            s = sel_np[b, g, :cnt_np[b, g]]
            o_ref, l_ref = oracle.sparse_attention(_q_ref(w, b, g), K, V, lens[b], w.P, s, w.tau)
            hs = slice(g * w.G, (g + 1) * w.G)
            assert_attn_close(out[b, hs], lse[b, hs], o_ref, l_ref)


def test_all_pages_equal_dense_attention(hz):
    w = SMALL["tiny"]
    announce("dense equivalence tiny")
    layer = hz.DeviceLayer(w, summaries=None)
    q = hz.queries_device(w)
    bufs = hz.StepBuffers(w.replace(k_fixed=w.Np))
    sel = torch.arange(w.Np, dtype=torch.int32).repeat(w.B, w.Hkv, 1).cuda()
    cnt = torch.full((w.B, w.Hkv), w.Np, dtype=torch.int32).cuda()
    hz.attend(layer, q, bufs, sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    out, lse = bufs.out.cpu().numpy(), bufs.lse.cpu().numpy()
    for g in range(w.Hkv):
        o_ref, l_ref = oracle.dense_attention(_q_ref(w, 0, g), wl.row_keys(w, 0, 0, g), wl.row_values(w, 0, 0, g), w.tau)
        assert_attn_close(out[0, g * w.G:(g + 1) * w.G], lse[0, g * w.G:(g + 1) * w.G], o_ref, l_ref)


def test_attention_edge_cases(hz):
    w = SMALL["llama_small"].replace(B=4)
    lens = [w.ctx, 0, 1, 17]
    announce(f"attention edges seq_lens={lens}")
    layer = hz.DeviceLayer(w, summaries=None, seq_lens=lens)
    qb = hz.queries_device(w)
    k = 5
    sel_np = np.full((w.B, w.Hkv, k), -1, np.int32)
    cnt_np = np.zeros((w.B, w.Hkv), np.int32)
    sel_np[0, :, :1] = 7                       # k = 1
    cnt_np[0] = 1
    sel_np[1, :, :2] = [0, 1]                  # empty sequence: skipped
    cnt_np[1] = 2
    sel_np[2, :, :3] = [0, 5, 9]               # only page 0 exists (one token)
    cnt_np[2] = 3
    sel_np[3, :, :2] = [1, 0]                  # unsorted is fine; page 1 partial (1 token)
    cnt_np[3] = 2
    bufs = hz.StepBuffers(w.replace(k_fixed=k))
    hz.attend(layer, qb, bufs, sel=torch.from_numpy(sel_np).cuda(), sel_count=torch.from_numpy(cnt_np).cuda())
    torch.cuda.synchronize()
    out, lse = bufs.out.cpu().numpy(), bufs.lse.cpu().numpy()
    for b in range(w.B):
        for g in range(w.Hkv):
            Np = oracle.num_pages(lens[b], w.P)
            s = [p for p in sel_np[b, g, :cnt_np[b, g]] if 0 <= p < Np]
            o_ref, l_ref = oracle.sparse_attention(_q_ref(w, b, g), wl.row_keys(w, 0, b, g),
                                                   wl.row_values(w, 0, b, g), lens[b], w.P, s, w.tau)
            hs = slice(g * w.G, (g + 1) * w.G)
            assert_attn_close(out[b, hs], lse[b, hs], o_ref, l_ref)
    assert np.all(out[1] == 0) and np.all(lse[1] == -np.inf)


# ---------------------------------------------------------------- summary builder

def check_page_summary(keys, rec, rank, counts):
    """One page's stored summary (rec: (1 + rank, d) float64 of the bf16
    record) against the oracle over its valid keys (n, d).

    The mean is unique: within half a bf16 ulp (plus slack).  The eigenvalues
    are unique, the eigenvectors only up to rotations inside a repeated (or
    nearly repeated) eigenvalue, so each kept w_j is checked by what holds for
    any valid choice: |w_j|^2 = lam_j (skipped within 1e-3 lam_1 of another
    eigenvalue), C w_j = lam_j w_j for the key covariance C = Xc^T Xc / n,
    w_i . w_j = 0 for i != j, and, where lam_R is clear of lam_{R+1}, the
    projector sum_j w_j w_j^T (= sum_j lam_j u_j u_j^T, unique then) against
    the oracle's.  Directions the oracle zeroes are zero."""
    n = keys.shape[0]
    mu, wv, lam, _ = oracle.summarize_page(keys, rank)
    mu_b = oracle.round_bf16(mu)
    ulp = np.maximum(np.abs(mu_b), 2.0 ** -126) * 2.0 ** -7
    assert np.all(np.abs(rec[0] - mu_b) <= ulp * 1.01)
    wg = rec[1:]
    Xc = keys.astype(np.float64) - mu
    C = Xc.T @ Xc / n
    lam_all = np.sort(np.linalg.eigvalsh(Xc @ Xc.T / n))[::-1]
    lam1 = lam_all[0]
    kept = [j for j in range(rank) if lam[j] != 0]
    for j in range(rank):
        if lam[j] == 0:
            assert not wg[j].any(), f"direction {j} should be zero (n = {n})"
            continue
        nw = np.linalg.norm(wg[j])
        assert np.linalg.norm(C @ wg[j] - lam[j] * wg[j]) <= 2e-2 * lam1 * nw, f"direction {j} is no eigenvector"
        for i in kept:
            if i < j:
                assert abs(wg[i] @ wg[j]) <= 1e-2 * lam1, f"directions {i}, {j} not orthogonal"
        gap_lo = lam_all[j - 1] - lam_all[j] if j > 0 else np.inf
        gap_hi = lam_all[j] - lam_all[j + 1] if j + 1 < len(lam_all) else np.inf
        if min(gap_lo, gap_hi) < 1e-3 * lam1:
            counts["skipped"] += 1
            continue
        counts["checked"] += 1
        assert abs(wg[j] @ wg[j] - lam[j]) <= 1e-2 * lam[j]
    cut = lam_all[rank - 1] - lam_all[rank] if rank < len(lam_all) else np.inf
    if cut >= 1e-3 * lam1 and lam1 > 0:
        Pg = wg.T @ wg
        Po = wv.T @ wv
        assert np.linalg.norm(Pg - Po) <= 2e-2 * np.linalg.norm(Po)
        counts["projectors"] += 1


def check_layer_summaries(w, layer, lens, row_keys, pages=None):
    rec = layer.summary.float().cpu().numpy().astype(np.float64).reshape(w.B, w.Hkv, w.Np, 1 + w.rank, w.d)
    log_n = layer.log_n.cpu().numpy()
    nv = layer.valid_tokens()
    counts = {"checked": 0, "skipped": 0, "projectors": 0}
    for b in range(w.B):
        Np = oracle.num_pages(lens[b], w.P)
        assert np.all(log_n[b, Np:] == -np.inf) and not rec[b, :, Np:].any()
        for g in range(w.Hkv):
            K = row_keys(b, g)
            for p in (range(Np) if pages is None else [p for p in pages if p < Np]):
                keys = K[p * w.P: min((p + 1) * w.P, lens[b])]
                n = keys.shape[0]
                assert nv[b, p] == n
                ln = log_n[b, p]
                assert ln == np.float32(math.log(n)) or abs(ln - math.log(n)) <= 2 ** -22 * max(1.0, math.log(n))
                check_page_summary(keys, rec[b, g, p], w.rank, counts)
    print(f"directions checked {counts['checked']}, skipped (near-degenerate) {counts['skipped']}, "
          f"projectors {counts['projectors']}")
    return counts


@pytest.mark.parametrize("name", ["tiny", "llama_small", "heavy_small", "gmm_small", "heavy_f16_small", "r8_p16",
                                  "r8_p32", "r1_p16"])
def test_summary_builder_invariants(hz, name):
    w = SMALL[name] if name in SMALL else SUMMARY_ONLY[name]
    lens = [w.ctx, w.ctx - w.P - 3] if w.B == 2 else [w.ctx]
    announce(f"summary build {name}")
    layer = hz.DeviceLayer(w, summaries="build", seq_lens=lens)
    torch.cuda.synchronize()
    counts = check_layer_summaries(w, layer, lens, lambda b, g: wl.row_keys(w, 0, b, g))
    assert counts["checked"] > 0


def crafted_page(kind, P, d, rng):
    """(P, d) float32 keys, exact in bfloat16 and float16, of a page whose
    spectrum is degenerate on purpose: keys +-a along a few coordinate axes
    (each axis gets as many + as - keys, so the centred keys are those
    offsets) on top of a shared random integer vector."""
    base = rng.integers(-3, 4, d).astype(np.float32)
    x = np.tile(base, (P, 1))
    def axes(amps):
        per = P // len(amps)
        for a, amp in enumerate(amps):
            for t in range(per):
                x[a * per + t, 5 + 7 * a] += amp * (1 if t % 2 == 0 else -1)
    if kind == "four_equal":          # one eigenvalue of multiplicity 4
        axes([2.0] * 4)
    elif kind == "two_pairs":         # two eigenvalues of multiplicity 2
        axes([3.0, 3.0, 2.0, 2.0])
    elif kind == "eight_equal":       # multiplicity 8: top-4 space not unique
        axes([2.0] * 8)
    elif kind == "rank_two":          # two non-zero eigenvalues, the rest zero
        axes([3.0, 2.0])
    elif kind == "identical":         # all keys equal: no spread
        pass
    elif kind == "doubled":           # random keys, each twice
        r = rng.integers(-4, 5, (P // 2, d)).astype(np.float32)
        x = np.repeat(r, 2, axis=0)
    return x


CRAFTED = ("four_equal", "two_pairs", "eight_equal", "rank_two", "identical", "doubled")


@pytest.mark.parametrize("name", ["llama_small", "heavy_small", "r8_p16", "r8_p32"])
def test_summary_builder_repeated_eigenvalues(hz, name):
    """Pages with repeated top eigenvalues, rank below R, no spread at all, and
    duplicated keys, written into the K pool and summarised again; a partial
    last page of each kind as well."""
    base = SMALL[name] if name in SMALL else SUMMARY_ONLY[name]
    w = base.replace(B=1, ctx=base.P * 40 + 6)
    lens = [w.ctx]
    announce(f"summary build on crafted pages {name}")
    layer = hz.DeviceLayer(w, summaries=None, seq_lens=lens)
    layer.summary = torch.empty((w.B, w.Hkv, w.Np, (1 + w.rank) * w.d), dtype=torch.bfloat16, device="cuda")
    rng = np.random.default_rng(7)
    dt = layer.k16.dtype
    pages = []
    for i, kind in enumerate(CRAFTED):
        for p in (3 + i, w.Np - 1 if i == 0 else 10 + i):
            phys = int(layer.bt_np[0, p])
            for g in range(w.Hkv):
                layer.k16[phys, g] = torch.from_numpy(crafted_page(kind, w.P, w.d, rng)).to(dt)
            pages.append(p)
    layer.build_summaries()
    torch.cuda.synchronize()
    pool = layer.k16.float().cpu().numpy()
    def row_keys(b, g):
        return pool[layer.bt_np[b], g].reshape(-1, w.d)
    counts = check_layer_summaries(w, layer, lens, row_keys, pages=sorted(set(pages)) + [0, 1, 2])
    assert counts["projectors"] > 0


# ---------------------------------------------------------------- codec

@pytest.mark.parametrize("shape", ["bf16_d128", "f16_d64", "fp8_bf16_d128", "fp8_f16_d64", "out_bf16_d128",
                                   "out_f16_d64"])
def test_pack_and_dequant_bit_exact(hz, shape):
    from quantized_kv_cache_summary_amd import kvsparse as kv
    base = W["tiers_fp8_64k"] if shape.startswith("fp8") else W["tiers_64k"]
    if shape.endswith("bf16_d128"):
        w = base.replace(B=2, ctx=16 * 96)
    else:
        w = base.replace(B=2, ctx=16 * 96, d=64, Hq=8, Hkv=2, dtype="f16", rank=2)
    outl = shape.startswith("out")
    announce(f"codec {shape}")
    layer = hz.DeviceLayer(w, summaries=None, b1_outliers=outl)
    k_all = layer.k16.view(torch.int16).cpu().numpy().view(np.uint16)
    v_all = layer.v16.view(torch.int16).cpu().numpy().view(np.uint16)
    present = sorted(set(w.tier_order) - {0})
    for t in present:
        phys = np.nonzero(layer.tier_phys == t)[0]
        assert phys.size > 0
        for src, codes, sz in ((k_all, layer.kq[t - 1], layer.ksz[t - 1]), (v_all, layer.vq[t - 1], layer.vsz[t - 1])):
            x = wl.bits_to_f32(src[phys], w.dtype)
            ref_codes, ref_sz = oracle.encode_vector(x, t)
            got_codes = codes[: phys.size].cpu().numpy()
            got_sz = sz[: phys.size].float().cpu().numpy()
            np.testing.assert_array_equal(got_codes, ref_codes)
            np.testing.assert_array_equal(got_sz, ref_sz)
        if outl and t == kv.KV_TIER_B1:
            for src, table in ((k_all, layer.kout), (v_all, layer.vout)):
                x = wl.bits_to_f32(src[phys], w.dtype)
                ref_words = oracle.encode_vector(x, t, outliers=True)[2]
                np.testing.assert_array_equal(table[: phys.size].cpu().numpy().view(np.uint32), ref_words)
    # standalone decode of every page through page_entry
    ids = torch.arange(w.n_phys, dtype=torch.int32).cuda()
    out = torch.empty((w.n_phys, 2, w.Hkv, w.P, w.d), dtype=torch.float32).cuda()
    kv.dequant_tier(layer.L, layer.pages, ids, out)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for t in [0] + present:
        phys = np.nonzero(layer.tier_phys == t)[0]
        for kvi, src in ((0, k_all), (1, v_all)):
            x = wl.bits_to_f32(src[phys], w.dtype)
            if t == 0:
                ref = x
            else:
                enc = oracle.encode_vector(x, t, outliers=outl)
                ref = oracle.decode_vector(enc[0], enc[1], t, w.d, outlier=enc[2] if len(enc) > 2 else None)
            np.testing.assert_array_equal(out[phys, kvi], ref)


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_fp8_every_code_ties_and_saturation(hz, dtype):
    """Crafted groups through kv_pack_tier and kv_dequant_tier: every finite
    E4M3 code (groups with max |x| = 448, so s = 1), the midpoints between
    neighbouring codes (ties to even), values past 448 after a rounded-down
    scale (saturation), signed zeros, and an all-zero group; codes, scales and
    decoded values bit-exact against the oracle."""
    from quantized_kv_cache_summary_amd import kvsparse as kv
    mags = oracle.e4m3_magnitudes()
    vals = np.concatenate([mags, -mags, (mags[:-1] + mags[1:]) / 2, -(mags[:-1] + mags[1:]) / 2, [-0.0]])
    groups = []
    for i in range(0, vals.size, 31):
        g = np.zeros(32)
        g[0] = 448.0
        chunk = vals[i:i + 31]
        g[1:1 + chunk.size] = chunk
        groups.append(g)
    g = np.zeros(32)
    g[:4] = [449.0, -449.0, 1.0, 300.0] if dtype == "f16" else [450.0, -450.0, 1.0, 300.0]
    groups.append(g)
    groups.append(np.zeros(32))
    d, P, Hkv = 128, 16, 1
    n_el = len(groups) * 32
    n_pages = -(-n_el // (P * d))
    x = np.zeros(n_pages * P * d)
    x[:n_el] = np.concatenate(groups)
    x32 = x.astype(np.float32)
    bits = wl.to_bits(x32, dtype)
    assert np.array_equal(wl.bits_to_f32(bits, dtype), x32)          # every crafted value is exact
    L = kv.layout(4, Hkv, d, P, 4, dtype)
    src = torch.from_numpy(bits.view(np.int16).reshape(n_pages, Hkv, P, d)).cuda()
    codes = torch.zeros((n_pages, Hkv, P, d), dtype=torch.uint8, device="cuda")
    sz = torch.zeros((n_pages, Hkv, P, d // 32, 2), dtype=torch.float16, device="cuda")
    announce(f"fp8 crafted groups {dtype}: {len(groups)} groups in {n_pages} pages")
    kv.pack_tier(L, src, n_pages, kv.KV_TIER_FP8, codes, sz)
    torch.cuda.synchronize()
    ref_c, ref_sz = oracle.encode_vector(x32.reshape(n_pages, Hkv, P, d), oracle.TIER_FP8)
    np.testing.assert_array_equal(codes.cpu().numpy(), ref_c)
    np.testing.assert_array_equal(sz.float().cpu().numpy(), ref_sz)
    assert set(range(256)) - set(np.unique(ref_c).tolist()) == {0x7F, 0xFF}   # every finite code occurs
    # decode through a page table with every page in the FP8 tier
    dummy8 = torch.zeros(16, dtype=torch.uint8, device="cuda")
    dummysz = torch.zeros(8, dtype=torch.float16, device="cuda")
    kq = [dummy8] * 4 + [codes]
    ksz = [dummysz] * 4 + [sz]
    entry = torch.from_numpy(((np.uint32(kv.KV_TIER_FP8) << np.uint32(29)) |
                              np.arange(n_pages, dtype=np.uint32)).view(np.int32)).cuda()
    pages = kv.make_pages(src, src, kq, kq, ksz, ksz, entry)
    out = torch.empty((n_pages, 2, Hkv, P, d), dtype=torch.float32, device="cuda")
    kv.dequant_tier(L, pages, torch.arange(n_pages, dtype=torch.int32, device="cuda"), out)
    torch.cuda.synchronize()
    ref = oracle.decode_vector(ref_c, ref_sz, oracle.TIER_FP8, d)
    got = out.cpu().numpy()
    for kvi in (0, 1):
        np.testing.assert_array_equal(got[:, kvi].view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("name,outl", [("tiers_64k", False), ("tiers_fp8_64k", False), ("tiers_64k", True)])
def test_tiered_attention_parity(hz, name, outl):
    w = W[name].replace(B=2, ctx=16 * 300)
    announce(f"tiered attention {name} outliers={outl}")
    layer = hz.DeviceLayer(w, summaries=None, b1_outliers=outl)
    q = hz.queries_device(w)
    k = w.k_of(w.Np)
    sel_np, cnt_np = wl.synthetic_selection(w, k)
    bufs = hz.StepBuffers(w)
    hz.attend(layer, q, bufs, sel=torch.from_numpy(sel_np).cuda(), sel_count=torch.from_numpy(cnt_np).cuda())
    torch.cuda.synchronize()
    out, lse = bufs.out.cpu().numpy(), bufs.lse.cpu().numpy()
    tiers = wl.page_tiers(w)
    for b in range(w.B):
        for g in range(w.Hkv):
            K = reconstruct_tiers(wl.row_keys(w, 0, b, g), w.ctx, w.P, tiers[b], b1_outliers=outl)
            V = reconstruct_tiers(wl.row_values(w, 0, b, g), w.ctx, w.P, tiers[b], b1_outliers=outl)
            o_ref, l_ref = oracle.sparse_attention(_q_ref(w, b, g), K, V, w.ctx, w.P, sel_np[b, g], w.tau)
            hs = slice(g * w.G, (g + 1) * w.G)
            assert_attn_close(out[b, hs], lse[b, hs], o_ref, l_ref)


# ---------------------------------------------------------------- whole step

def test_end_to_end_tiny_selects_planted_pages(hz):
    w = W["tiny"]
    announce("end to end tiny")
    layer = hz.DeviceLayer(w, summaries="build")
    q = hz.queries_device(w)
    bufs = hz.StepBuffers(w, with_S=True)
    hz.decode_step(layer, q, bufs)
    torch.cuda.synchronize()
    sel = bufs.sel.cpu().numpy()
    out, lse = bufs.out.cpu().numpy(), bufs.lse.cpu().numpy()
    hot = set(wl.hot_pages(w, 0, 0).tolist())
    for g in range(w.Hkv):
        r = oracle.decode_row(_q_ref(w, 0, g), wl.row_keys(w, 0, 0, g), wl.row_values(w, 0, 0, g), w.ctx, w.P,
                              w.rank, w.tau, k_fixed=w.k_fixed)
        assert hot <= set(sel[0, g].tolist())
        # the builder differs from the oracle's only by float32 eigen-solver rounding,
        # which moves scores by far less than the band used here
        check_selection(r["S"], w.k_fixed, sel[0, g], rel=1e-3)
        if set(sel[0, g].tolist()) == set(r["sel"].tolist()):
            hs = slice(g * w.G, (g + 1) * w.G)
            assert_attn_close(out[0, hs], lse[0, hs], r["out"], r["lse"])


def test_determinism(hz):
    w = SMALL["qwen_small"]
    announce("determinism")
    layer = hz.DeviceLayer(w, summaries="build")
    q = hz.queries_device(w)
    res = []
    for _ in range(2):
        bufs = hz.StepBuffers(w, with_S=True)
        hz.decode_step(layer, q, bufs)
        torch.cuda.synchronize()
        res.append([t.cpu().numpy().copy() for t in (bufs.head_scores, bufs.page_S, bufs.sel, bufs.out, bufs.lse)])
    for a, b in zip(*res):
        assert np.array_equal(a, b, equal_nan=True)


def test_nan_query_ranks_as_minus_inf(hz):
    w = SMALL["tiny"]
    announce("nan query")
    layer = hz.DeviceLayer(w, summaries="build")
    q = hz.queries_device(w)
    q[0, 0, 3] = float("nan")                      # one head of KV group 0
    bufs = hz.StepBuffers(w, with_S=True)
    hz.decode_step(layer, q, bufs)
    torch.cuda.synchronize()
    sel = bufs.sel.cpu().numpy()
    assert list(sel[0, 0]) == list(range(w.k_fixed))     # all S NaN -> lowest indices
    out = bufs.out.cpu().numpy()
    assert np.isnan(out[0, 0]).all()
    assert not np.isnan(out[0, w.G:]).any()


def test_out_of_range_device_values():
    """Values read from device memory are not checked on the host; the calls
    clamp or skip them as documented.  A sequence length past max_pages * P
    gives the same step as the full length (bit for bit), a negative one the
    same as an empty row; selection entries outside [0, Np) are skipped and a
    count above k_max is clamped (attention within float32 rounding of the
    call on the valid entries alone: the dealing of pages to waves changes)."""
    from quantized_kv_cache_summary_amd import harness as hz
    from quantized_kv_cache_summary_amd import kvsparse as kv
    w = W["llama8b_32k"].replace(B=3, ctx=16 * 200)
    announce("out-of-range sequence lengths and selection entries")
    layer = hz.DeviceLayer(w, summaries="synthetic", seq_lens=[w.ctx, 0, w.ctx - 37])
    q = hz.queries_device(w)
    ref = hz.StepBuffers(w, with_S=True)
    hz.whole_step(layer, q, ref)
    good = layer.seq_lens.clone()
    layer.seq_lens = torch.tensor([w.ctx + 1000, -5, w.ctx - 37], dtype=torch.int32, device="cuda")
    odd = hz.StepBuffers(w, with_S=True)
    hz.whole_step(layer, q, odd)
    layer.seq_lens = good
    torch.cuda.synchronize()
    for name in ("sel", "sel_count"):
        np.testing.assert_array_equal(getattr(odd, name).cpu().numpy(), getattr(ref, name).cpu().numpy())
    for name in ("head_scores", "out", "lse"):
        np.testing.assert_array_equal(getattr(odd, name).cpu().numpy().view(np.uint32),
                                      getattr(ref, name).cpu().numpy().view(np.uint32))
    assert np.all(odd.out.cpu().numpy()[1] == 0) and np.all(np.isneginf(odd.lse.cpu().numpy()[1]))

    # attention over a selection with invalid entries and an oversized count
    k_max = ref.sel.shape[-1]
    sel = ref.sel.clone()
    cnt = ref.sel_count.clone()
    k0 = int(cnt[0, 0].item())
    sel[0, 0, 1] = -1
    sel[0, 0, 3] = w.Np + 7
    bad = torch.tensor([int(sel[0, 0, 1].item()), int(sel[0, 0, 3].item())])
    assert bad.tolist() == [-1, w.Np + 7]
    cnt[0, 1] = k_max + 50                       # clamped to k_max; entries past the row's k are -1
    out_a = torch.empty_like(ref.out)
    lse_a = torch.empty_like(ref.lse)
    kv.sparse_decode_attn(layer.L, q, layer.pages, layer.bt, layer.seq_lens, sel, cnt, out_a, lse_a, ref.ws)
    # the same attention on the valid entries alone
    keep = [i for i in range(k0) if i not in (1, 3)]
    sel_b = ref.sel.clone()
    cnt_b = ref.sel_count.clone()
    sel_b[0, 0, :len(keep)] = ref.sel[0, 0, keep]
    sel_b[0, 0, len(keep):] = -1
    cnt_b[0, 0] = len(keep)
    out_b = torch.empty_like(ref.out)
    lse_b = torch.empty_like(ref.lse)
    kv.sparse_decode_attn(layer.L, q, layer.pages, layer.bt, layer.seq_lens, sel_b, cnt_b, out_b, lse_b, ref.ws)
    torch.cuda.synchronize()
    np.testing.assert_allclose(out_a.cpu().numpy(), out_b.cpu().numpy(), rtol=0, atol=1e-5)
    np.testing.assert_allclose(lse_a.cpu().numpy(), lse_b.cpu().numpy(), rtol=0, atol=1e-5)
    layer.release()
