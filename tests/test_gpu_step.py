"""GPU parity of the whole-step call (kv_sparse_decode_step: score, then the
fused selector + attention or the separate selector and attention launches).

The step must write every output bit for bit as kv_page_score followed by
kv_topk_sparse_decode_attn with the same arguments and split count (head
scores, score partials, sel, sel_count, page_S, out, lse), leave its
workspace's counters at zero, and match the oracle to the usual bars:
scores within 1e-5 relative on the stored summary, band-exact selection against
the oracle's S, attention within 2e-3 over the selected pages.  Covered:
ragged rows and rows whose page count is not a multiple of the score item,
every split-count shape, d = 64 and 128, ranks 1 / 4 / 8, float16 and
bfloat16, page sizes 16 and 32, 4 and 8 query heads per KV head, packed tiers
(with FP8), an odd number of rows, empty / one-token / short rows, forced pages,
k_fixed, keep = 1, coverage mode, calls in a row on one workspace, HIP graph
replays, a host-mapped value pool with a hot buffer, and the full workload
size the benchmark times.
"""

import numpy as np
import pytest
import torch

import oracle
from parity import assert_attn_close, assert_scores_close, bits_to_f64, check_selection
from quantized_kv_cache_summary_amd import workloads as wl

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS
SMALL = {
    "tiny": W["tiny"],
    "llama_small": W["llama8b_32k"].replace(B=2, ctx=16 * 300 + 7),
    "llama_r8_f16": W["llama8b_32k"].replace(B=2, ctx=16 * 200 + 3, rank=8, dtype="f16"),
    "tiny_r1_long": W["tiny"].replace(B=3, ctx=16 * 150 + 9, rank=1),
    "heavy_g4": W["heavy70b_128k"].replace(B=2, Hq=8, Hkv=2, ctx=32 * 150 + 5, v_host=False),
    "qwen_small": W["qwen3b_128k"].replace(B=2, ctx=16 * 400 + 9),
    "tiers_small": W["tiers_64k"].replace(B=2, ctx=16 * 300),
    "tiers_fp8_small": W["tiers_fp8_64k"].replace(B=3, ctx=16 * 250 + 1),
}


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def hz():
    from quantized_kv_cache_summary_amd import harness
    return harness


@pytest.fixture(scope="module")
def kv():
    from quantized_kv_cache_summary_amd import kvsparse
    return kvsparse


def _bits(t):
    return t.cpu().numpy().view(np.uint32)


def _ragged(w):
    return [w.ctx] + [max(1, w.ctx - (3 + 2 * i) * w.P - 5) for i in range(1, w.B)]


def _ws_counters(bufs, w):
    """The workspace's per-row split counters (its first B * Hkv words; zero between calls)."""
    return bufs.ws.view(torch.int32)[:w.rows].cpu().numpy()


def _reference(hz, layer, q, w, splits, **sel_args):
    a = hz.StepBuffers(w, num_splits=splits, with_S=True)
    a.page_S.zero_()              # entries past a row's pages are never written
    hz.score(layer, q, a)
    hz.topk_attend(layer, q, a, **sel_args)
    return a


def _step(hz, layer, q, w, splits, bufs=None, **sel_args):
    f = bufs or hz.StepBuffers(w, num_splits=splits, with_S=True)
    f.sel.fill_(-7)
    f.sel_count.fill_(-7)
    f.page_S.zero_()
    f.head_scores.fill_(float("nan"))
    f.lse_partial.fill_(float("nan"))
    hz.whole_step(layer, q, f, **sel_args)
    return f


def _assert_same(a, f):
    np.testing.assert_array_equal(_bits(f.head_scores), _bits(a.head_scores))
    np.testing.assert_array_equal(_bits(f.lse_partial), _bits(a.lse_partial))
    np.testing.assert_array_equal(f.sel_count.cpu().numpy(), a.sel_count.cpu().numpy())
    np.testing.assert_array_equal(f.sel.cpu().numpy(), a.sel.cpu().numpy())
    np.testing.assert_array_equal(_bits(f.page_S), _bits(a.page_S))
    np.testing.assert_array_equal(_bits(f.out), _bits(a.out))
    np.testing.assert_array_equal(_bits(f.lse), _bits(a.lse))


def _assert_ws_clean(kv, bufs, w, L):
    ctr = _ws_counters(bufs, w)
    assert np.all(ctr == 0), f"workspace counters not reset: {np.nonzero(ctr)[0][:10]}"


@pytest.mark.parametrize("name", list(SMALL))
@pytest.mark.parametrize("splits", [0, 1, 3])
def test_step_equals_score_and_fused(hz, kv, name, splits):
    w = SMALL[name]
    lens = _ragged(w)
    announce(f"step vs score + fused {name} splits={splits} seq_lens={lens}")
    layer = hz.DeviceLayer(w, summaries="synthetic", seq_lens=lens)
    q = hz.queries_device(w)
    a = _reference(hz, layer, q, w, splits)
    f = _step(hz, layer, q, w, splits)
    torch.cuda.synchronize()
    assert hz.step_supported(layer, f)
    _assert_same(a, f)
    _assert_ws_clean(kv, f, w, layer.L)


@pytest.mark.parametrize("name", ["llama_small", "llama_r8_f16", "tiny_r1_long", "heavy_g4", "qwen_small"])
def test_step_matches_oracle(hz, name):
    """Scores, selection and attention of the step against the oracle."""
    w = SMALL[name]
    lens = _ragged(w)
    announce(f"step vs oracle {name} seq_lens={lens}")
    layer = hz.DeviceLayer(w, summaries="synthetic", seq_lens=lens)
    f = _step(hz, layer, hz.queries_device(w), w, 0)
    torch.cuda.synchronize()
    hs = f.head_scores.cpu().numpy().astype(np.float64)
    sel, cnt = f.sel.cpu().numpy(), f.sel_count.cpu().numpy()
    S_gpu = f.page_S.cpu().numpy()
    out, lse = f.out.cpu().numpy(), f.lse.cpu().numpy()
    rec_bits, n_valid = wl.synthetic_summary(w)
    rec = bits_to_f64(rec_bits)
    log_n = np.log(n_valid.astype(np.float64)).astype(np.float32).astype(np.float64)
    for b in range(w.B):
        Np = oracle.num_pages(lens[b], w.P)
        for g in range(w.Hkv):
            qg = wl.queries(w, 0, b, g).astype(np.float64)
            s_ref = oracle.page_score(qg, rec[b, g, :Np, 0], rec[b, g, :Np, 1:], log_n[b, :Np], w.tau)
            assert_scores_close(hs[b, g, :, :Np], s_ref, what="head scores")
            S_ref = oracle.group_aggregate(s_ref)
            assert_scores_close(S_gpu[b, g, :Np], S_ref, what="S")
            k = oracle.selection_count(Np, w.keep, w.k_fixed)
            assert cnt[b, g] == k
            check_selection(S_ref, k, sel[b, g, :k])
            assert np.all(sel[b, g, k:] == -1)
            o_ref, l_ref = oracle.sparse_attention(qg, wl.row_keys(w, 0, b, g), wl.row_values(w, 0, b, g),
                                                   lens[b], w.P, sel[b, g, :k], w.tau)
            heads = slice(g * w.G, (g + 1) * w.G)
            assert_attn_close(out[b, heads], lse[b, heads], o_ref, l_ref)


@pytest.mark.parametrize("name", ["llama_small", "qwen_small", "tiers_small"])
def test_step_edge_rows_and_selection_modes(hz, kv, name):
    """Empty, one-token and short rows beside a long one; forced pages,
    k_fixed and keep = 1, each against score + fused bit for bit, through the
    fused schedule (llama_small) and the separate one (G = 8, packed tiers)."""
    base = SMALL[name].replace(B=4)
    lens = [base.ctx, 0, 1, 17]
    for keep, k_fixed, nff, nfl in ((base.keep, 0, 0, 0), (base.keep, 0, 2, 3), (0.0, 5, 1, 1), (1.0, 0, 0, 0)):
        w = base.replace(keep=keep, k_fixed=k_fixed)
        announce(f"step edge rows {name} seq_lens={lens} keep={keep} k_fixed={k_fixed} forced=({nff},{nfl})")
        layer = hz.DeviceLayer(w, summaries="synthetic", seq_lens=lens)
        q = hz.queries_device(w)
        a = _reference(hz, layer, q, w, 0, n_force_first=nff, n_force_last=nfl)
        f = _step(hz, layer, q, w, 0, n_force_first=nff, n_force_last=nfl)
        torch.cuda.synchronize()
        _assert_same(a, f)
        _assert_ws_clean(kv, f, w, layer.L)
        assert np.all(f.out.cpu().numpy()[1] == 0) and np.all(f.lse.cpu().numpy()[1] == -np.inf)
        assert np.all(f.sel_count.cpu().numpy()[1] == 0)


@pytest.mark.parametrize("name", ["llama_small", "qwen_small", "tiers_small"])
@pytest.mark.parametrize("coverage", [0.5, 0.95])
def test_step_coverage_mode(hz, kv, coverage, name):
    w = SMALL[name]
    lens = _ragged(w)
    announce(f"step coverage={coverage} {name} seq_lens={lens}")
    layer = hz.DeviceLayer(w, summaries="synthetic", seq_lens=lens)
    q = hz.queries_device(w)
    res = []
    for one in (False, True):
        bufs = hz.StepBuffers(w, with_S=True)
        # the selection's row length is the cap in coverage mode
        bufs.sel = torch.full((w.B, w.Hkv, w.Np), -7, dtype=torch.int32, device="cuda")
        bufs.ws = torch.zeros(max(1, kv.attn_workspace_size(layer.L, w.B, w.Np) // 4), dtype=torch.float32,
                              device="cuda")
        bufs.page_S.zero_()
        if one:
            bufs = _step(hz, layer, q, w, 0, bufs=bufs, coverage=coverage)
        else:
            hz.score(layer, q, bufs)
            hz.topk_attend(layer, q, bufs, coverage=coverage)
        torch.cuda.synchronize()
        res.append(bufs)
    _assert_same(res[0], res[1])
    cnt = res[1].sel_count.cpu().numpy()
    if name == "llama_small":    # N(0,1) keys: coverage keeps more than the 8 % budget here
        assert np.all(cnt > oracle.selection_count(w.Np, w.keep, 0))
    _assert_ws_clean(kv, res[1], w, layer.L)


def test_step_calls_in_a_row_and_graph_replays(hz, kv):
    """Several calls on one workspace, then a captured graph replayed with
    eager work between replays: every result equals its own reference."""
    w = SMALL["llama_small"]
    lens = _ragged(w)
    announce(f"step calls in a row and graph replays seq_lens={lens}")
    layer = hz.DeviceLayer(w, summaries="synthetic", seq_lens=lens)
    qs = [hz.queries_device(w, qidx=i) for i in range(3)]
    f = hz.StepBuffers(w, with_S=True)
    for q in qs:
        a = _reference(hz, layer, q, w, 0)
        _step(hz, layer, q, w, 0, bufs=f)
        torch.cuda.synchronize()
        _assert_same(a, f)
        _assert_ws_clean(kv, f, w, layer.L)
    qbuf = qs[0].clone()
    g = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        hz.whole_step(layer, qbuf, f)          # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(g):
        hz.whole_step(layer, qbuf, f)
    torch.cuda.synchronize()
    for i in (1, 2, 0, 1):
        qbuf.copy_(qs[i])
        a = _reference(hz, layer, qs[i], w, 0)      # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _assert_same(a, f)
        _assert_ws_clean(kv, f, w, layer.L)


def test_step_host_mapped_values_with_hot_buffer(hz, kv):
    w = W["heavy70b_128k"].replace(B=2, Hq=8, Hkv=2, ctx=32 * 150 + 5)     # V in mapped host memory
    announce("step with host-mapped V and a warm hot buffer")
    layer = hz.DeviceLayer(w, summaries="synthetic", hot_mode="warm")
    try:
        q = hz.queries_device(w)
        a = _reference(hz, layer, q, w, 0)
        f = _step(hz, layer, q, w, 0)
        torch.cuda.synchronize()
        _assert_same(a, f)
        _assert_ws_clean(kv, f, w, layer.L)
    finally:
        layer.release()


@pytest.mark.timeout(600)
def test_step_full_size(hz, kv):
    """The full 8 x 32 K workload in the launch configuration the benchmark
    times: bit for bit against score + fused, sampled rows against the oracle."""
    w = W["llama8b_32k"]
    announce("step full size llama8b_32k")
    layer = hz.DeviceLayer(w, summaries="synthetic")
    q = hz.queries_device(w)
    a = _reference(hz, layer, q, w, 0)
    f = _step(hz, layer, q, w, 0)
    torch.cuda.synchronize()
    _assert_same(a, f)
    _assert_ws_clean(kv, f, w, layer.L)
    sel, cnt = f.sel.cpu().numpy(), f.sel_count.cpu().numpy()
    out, lse = f.out.cpu().numpy(), f.lse.cpu().numpy()
    rec_bits, n_valid = wl.synthetic_summary(w)
    log_n = np.log(n_valid.astype(np.float64)).astype(np.float32).astype(np.float64)
    for b, g in [(b, g) for b in range(w.B) for g in range(w.Hkv)]:       # all 64 rows
        rec = bits_to_f64(rec_bits[b, g])
        qg = wl.queries(w, 0, b, g).astype(np.float64)
        S_ref = oracle.group_aggregate(oracle.page_score(qg, rec[:, 0], rec[:, 1:], log_n[b], w.tau))
        k = oracle.selection_count(w.Np, w.keep, w.k_fixed)
        assert cnt[b, g] == k
        check_selection(S_ref, k, sel[b, g, :k])
        o_ref, l_ref = oracle.sparse_attention(qg, wl.row_keys(w, 0, b, g), wl.row_values(w, 0, b, g), w.ctx, w.P,
                                               sel[b, g, :k], w.tau)
        heads = slice(g * w.G, (g + 1) * w.G)
        assert_attn_close(out[b, heads], lse[b, heads], o_ref, l_ref)


@pytest.mark.parametrize("name", ["llama_small", "qwen_small", "tiers_small"])
@pytest.mark.parametrize("coverage,nff,nfl", [(0.5, 0, 0), (0.95, 0, 0), (0.8, 2, 3)])
def test_step_coverage_matches_oracle(hz, name, coverage, nff, nfl):
    """A coverage-mode step (selection by attention-mass coverage, then the
    attention) against the oracle's decode of each row on the same stored
    summary: k within the counts for coverages +-1e-5, the set band-exact, and
    the attention within 2e-3 (over the oracle's own set where the two agree,
    else over the GPU's set)."""
    w = SMALL[name]
    lens = _ragged(w)
    announce(f"step coverage={coverage} forced=({nff},{nfl}) vs oracle {name} seq_lens={lens}")
    layer = hz.DeviceLayer(w, summaries="synthetic", seq_lens=lens)
    q = hz.queries_device(w)
    bufs = hz.StepBuffers(w, with_S=True)
    bufs.sel = torch.full((w.B, w.Hkv, w.Np), -7, dtype=torch.int32, device="cuda")   # cap = Np
    bufs.ws = torch.zeros(max(1, hz.kv.attn_workspace_size(layer.L, w.B, w.Np) // 4), dtype=torch.float32,
                          device="cuda")
    f = _step(hz, layer, q, w, 0, bufs=bufs, coverage=coverage, n_force_first=nff, n_force_last=nfl)
    torch.cuda.synchronize()
    sel, cnt = f.sel.cpu().numpy(), f.sel_count.cpu().numpy()
    out, lse = f.out.cpu().numpy(), f.lse.cpu().numpy()
    rec_bits, n_valid = wl.synthetic_summary(w)
    rec = bits_to_f64(rec_bits)
    log_n = np.log(n_valid.astype(np.float64)).astype(np.float32).astype(np.float64)
    tiers = wl.page_tiers(w)
    same = 0
    for b in range(w.B):
        Np = oracle.num_pages(lens[b], w.P)
        for g in range(w.Hkv):
            qg = wl.queries(w, 0, b, g).astype(np.float64)
            r = oracle.decode_row(qg, wl.row_keys(w, 0, b, g), wl.row_values(w, 0, b, g), lens[b], w.P, w.rank,
                                  w.tau, n_force_first=nff, n_force_last=nfl,
                                  page_tiers=None if tiers is None else tiers[b],
                                  summary=(rec[b, g, :Np, 0], rec[b, g, :Np, 1:], log_n[b, :Np]),
                                  coverage=coverage, k_cap=w.Np)
            k = int(cnt[b, g])
            lo = oracle.coverage_count(r["S"], max(0.0, coverage - 1e-5), w.Np, nff, nfl)
            hi = oracle.coverage_count(r["S"], coverage + 1e-5, w.Np, nff, nfl)
            assert lo <= r["k"] <= hi and lo <= k <= hi, (b, g, k, r["k"], lo, hi)
            forced = [p for p in range(Np) if p < nff or p >= Np - nfl]
            check_selection(r["S"], k, sel[b, g, :k], forced=forced)
            assert np.all(sel[b, g, k:] == -1)
            heads = slice(g * w.G, (g + 1) * w.G)
            if k == r["k"] and np.array_equal(sel[b, g, :k], r["sel"]):
                same += 1
                assert_attn_close(out[b, heads], lse[b, heads], r["out"], r["lse"])
            else:
                K, V = wl.row_keys(w, 0, b, g), wl.row_values(w, 0, b, g)
                if tiers is not None:
                    K = oracle.pipeline.reconstruct_tiers(K, lens[b], w.P, tiers[b])
                    V = oracle.pipeline.reconstruct_tiers(V, lens[b], w.P, tiers[b])
                o_ref, l_ref = oracle.sparse_attention(qg, K, V, lens[b], w.P, sel[b, g, :k], w.tau)
                assert_attn_close(out[b, heads], lse[b, heads], o_ref, l_ref)
    print(f"rows whose set equals the oracle's: {same} of {w.rows}")
    assert same >= 1
