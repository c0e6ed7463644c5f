"""GPU parity of the r8 low-rank score (kv_lowrank_coords,
kv_page_score_lowrank, the row mean of kv_basis_build) against the oracle, at
small sizes with ragged rows and sampled full-size rows.

* score + select from seeded stored state (basis, mean, bf16 coordinates):
  every row element-wise (1e-5 relative), selections band-exact;
* coordinates from the real keys with a seeded basis and mean given to both
  sides: within one bf16 ulp of the oracle's plus the float32 dot product's
  error bound (fp32 against fp64 before the rounding);
* the row mean from kv_basis_build within float32 rounding of the oracle's;
* end to end (coordinates built on the GPU from the seeded basis): selection
  within a relaxed band and attention within 2e-3 where the sets agree.
"""

import numpy as np
import pytest
import torch

import oracle
from parity import assert_scores_close, check_selection, assert_attn_close, bits_to_f64
from quantized_kv_cache_summary_amd import workloads as wl

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS
SMALL = {
    "tiny": W["tiny"],
    "llama_small": W["llama8b_32k"].replace(B=2, ctx=16 * 300 + 7),
    "qwen_small": W["qwen3b_128k"].replace(B=2, ctx=16 * 400),             # G = 8
    "heavy_small": W["heavy70b_128k"].replace(B=2, Hq=16, Hkv=2, ctx=32 * 150 + 5, v_host=False),  # P = 32
    "g16_small": W["llama8b_32k"].replace(B=2, Hq=32, Hkv=2, ctx=16 * 100 + 3),                   # G = 16
}


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def hz():
    from quantized_kv_cache_summary_amd import harness
    return harness


def _lens(w):
    return [w.ctx, max(1, w.ctx - 3 * w.P - 5)] if w.B == 2 else [w.ctx]


def _stored(w, lens):
    U, m, cbits = wl.synthetic_lowrank(w, 0, seq_lens_=lens)
    return U.astype(np.float64), m.astype(np.float64), bits_to_f64(cbits)


def _row_scores(w, b, g, U, m, C, L):
    qg = wl.queries(w, 0, b, g).astype(np.float64)
    return oracle.page_score_lowrank(qg, C[b, g].reshape(-1, C.shape[-1]), m[b, g], U[b, g], L, w.P, w.tau)


@pytest.mark.parametrize("name", list(SMALL))
def test_lowrank_score_and_select_parity(hz, name):
    w = SMALL[name]
    lens = _lens(w)
    announce(f"r8 score/select {name} seq_lens={lens}")
    layer = hz.DeviceLayer(w, summaries="lowrank_synthetic", seq_lens=lens)
    q = hz.queries_device(w)
    bufs = hz.StepBuffers(w, with_S=True)
    hz.score(layer, q, bufs)
    hz.topk(layer, bufs)
    torch.cuda.synchronize()
    hs, S_gpu, sel = bufs.head_scores.cpu().numpy(), bufs.page_S.cpu().numpy(), bufs.sel.cpu().numpy()
    U, m, C = _stored(w, lens)
    for b in range(w.B):
        Np = oracle.num_pages(lens[b], w.P)
        for g in range(w.Hkv):
            s_ref = _row_scores(w, b, g, U, m, C, lens[b])
            assert_scores_close(hs[b, g, :, :Np], s_ref)
            assert np.all(hs[b, g, :, Np:] == -np.inf)
            S_ref = oracle.group_aggregate(s_ref)
            assert_scores_close(S_gpu[b, g, :Np], S_ref, what="S")
            k = oracle.selection_count(Np, w.keep, w.k_fixed)
            check_selection(S_ref, k, sel[b, g, :k])


@pytest.mark.parametrize("name", ["tiny", "llama_small", "heavy_small"])
def test_lowrank_coordinates_parity(hz, name):
    from quantized_kv_cache_summary_amd import kvsparse as kv
    w = SMALL[name]
    lens = _lens(w)
    announce(f"r8 coordinates {name}")
    layer = hz.DeviceLayer(w, summaries="lowrank_synthetic", seq_lens=lens)
    layer.coords.zero_()
    entries, nv = layer._all_entries()
    kv.lowrank_coords(layer.L_lr, layer.k_src, layer.bt, entries, nv, layer.lr_basis, layer.lr_mean, layer.coords)
    torch.cuda.synchronize()
    got = layer.coords.float().cpu().numpy().astype(np.float64)
    U, m, _ = _stored(w, lens)
    worst = 0
    for b in range(w.B):
        for g in range(w.Hkv):
            K = wl.row_keys(w, 0, b, g)[: lens[b]]
            ref = oracle.key_coords(K, U[b, g], m[b, g])
            gr = got[b, g].reshape(-1, ref.shape[1])[: lens[b]]
            # one bf16 ulp of the result, plus the float32 dot product's own
            # error (d terms, each rounding at most 2^-24 of the running sum)
            ulp = np.maximum(np.abs(ref), 2.0 ** -126) * 2.0 ** -7
            acc = (np.abs(K.astype(np.float64) - m[b, g]) @ np.abs(U[b, g]).T) * (w.d * 2.0 ** -24)
            assert np.all(np.abs(gr - ref) <= ulp * 1.01 + acc), (b, g)
            worst = max(worst, int(np.sum(gr != ref)))
            assert not got[b, g].reshape(-1, ref.shape[1])[lens[b]:].any()
    print(f"coordinates one ulp apart: {worst}")


@pytest.mark.parametrize("name", ["tiny", "llama_small"])
def test_basis_build_row_mean(hz, name):
    from quantized_kv_cache_summary_amd import kvsparse as kv
    w = SMALL[name]
    lens = _lens(w)
    announce(f"row mean from the basis build {name}")
    layer = hz.DeviceLayer(w, summaries="lowrank_build", seq_lens=lens)
    torch.cuda.synchronize()
    mean = layer.lr_mean.cpu().numpy().astype(np.float64)
    for b in range(w.B):
        for g in range(w.Hkv):
            ref = oracle.row_mean(wl.row_keys(w, 0, b, g)[: lens[b]])
            np.testing.assert_allclose(mean[b, g], ref, rtol=0, atol=2e-6 * (1 + np.abs(ref).max()))


@pytest.mark.parametrize("name", ["tiny", "llama_small", "qwen_small"])
def test_lowrank_end_to_end_seeded_basis(hz, name):
    from quantized_kv_cache_summary_amd import kvsparse as kv
    w = SMALL[name]
    lens = _lens(w)
    announce(f"r8 end to end {name}")
    layer = hz.DeviceLayer(w, summaries="lowrank_synthetic", seq_lens=lens)
    entries, nv = layer._all_entries()
    kv.lowrank_coords(layer.L_lr, layer.k_src, layer.bt, entries, nv, layer.lr_basis, layer.lr_mean, layer.coords)
    q = hz.queries_device(w)
    bufs = hz.StepBuffers(w)
    hz.decode_step(layer, q, bufs)
    torch.cuda.synchronize()
    U, m, _ = _stored(w, lens)
    sel, out, lse = bufs.sel.cpu().numpy(), bufs.out.cpu().numpy(), bufs.lse.cpu().numpy()
    compared = 0
    for b in range(w.B):
        for g in range(w.Hkv):
            K = wl.row_keys(w, 0, b, g)
            Cref = oracle.key_coords(K[: lens[b]], U[b, g], m[b, g])
            qg = wl.queries(w, 0, b, g).astype(np.float64)
            s_ref = oracle.page_score_lowrank(qg, Cref, m[b, g], U[b, g], lens[b], w.P, w.tau)
            S_ref = oracle.group_aggregate(s_ref)
            Np = oracle.num_pages(lens[b], w.P)
            k = oracle.selection_count(Np, w.keep, w.k_fixed)
            check_selection(S_ref, k, sel[b, g, :k], rel=1e-3)
            ref_sel = oracle.select_pages(S_ref, k)
            if set(sel[b, g, :k].tolist()) == set(ref_sel.tolist()):
                o_ref, l_ref = oracle.sparse_attention(qg, K, wl.row_values(w, 0, b, g), lens[b], w.P, ref_sel,
                                                       w.tau)
                hs = slice(g * w.G, (g + 1) * w.G)
                assert_attn_close(out[b, hs], lse[b, hs], o_ref, l_ref)
                compared += 1
    assert compared >= 1


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name", ["llama8b_32k", "qwen3b_128k"])
def test_lowrank_full_size_score_select(hz, name):
    w = W[name]
    announce(f"full size {name}: r8 score/select on seeded state")
    layer = hz.DeviceLayer(w, summaries="lowrank_synthetic")
    q = hz.queries_device(w)
    bufs = hz.StepBuffers(w, with_S=True)
    hz.score(layer, q, bufs)
    hz.topk(layer, bufs)
    torch.cuda.synchronize()
    lens = wl.seq_lens(w)
    U, m, C = _stored(w, lens)
    for b, g in [(0, 0), (w.B // 2, w.Hkv - 1), (w.B - 1, w.Hkv // 2)]:
        s_ref = _row_scores(w, b, g, U, m, C, int(lens[b]))
        assert_scores_close(bufs.head_scores[b, g].cpu().numpy(), s_ref)
        S_ref = oracle.group_aggregate(s_ref)
        assert_scores_close(bufs.page_S[b, g].cpu().numpy(), S_ref, what="S")
        k = oracle.selection_count(w.Np, w.keep, w.k_fixed)
        check_selection(S_ref, k, bufs.sel[b, g, :k].cpu().numpy())
