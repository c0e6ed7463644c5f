"""The whole-step call that allocates nothing (kv_sparse_decode_step_noalloc)
against kv_sparse_decode_step with a caller workspace: every output bit for bit,
on calls in a row over different numbers of rows (the second call smaller),
native and packed pages, and inside a captured HIP graph replayed with eager
work between replays."""

import numpy as np
import pytest
import torch

from quantized_kv_cache_summary_amd import workloads as wl

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS


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


def _outputs(f):
    return [_bits(f.head_scores), _bits(f.lse_partial), f.sel.cpu().numpy(), f.sel_count.cpu().numpy(),
            _bits(f.page_S), _bits(f.out), _bits(f.lse)]


def _fresh(hz, w, splits):
    f = hz.StepBuffers(w, num_splits=splits, with_S=True)
    f.sel.fill_(-7)
    f.sel_count.fill_(-7)
    f.page_S.zero_()
    f.head_scores.fill_(float("nan"))
    f.lse_partial.fill_(float("nan"))
    f.out.fill_(float("nan"))
    f.lse.fill_(float("nan"))
    return f


def _noalloc(kv, layer, q, f, stream=None, **sel):
    w = layer.w
    kv.sparse_decode_step_noalloc(layer.L, q, layer.summary, layer.log_n, layer.pages, layer.bt, layer.seq_lens,
                                  f.head_scores, f.lse_partial, f.sel, f.sel_count, f.out, f.lse, keep_frac=w.keep,
                                  k_fixed=w.k_fixed, page_S=f.page_S, num_splits=f.num_splits, stream=stream, **sel)


CASES = [
    # (workload, seq_lens offsets, splits, selection arguments)
    (W["llama8b_32k"].replace(B=3, ctx=16 * 300 + 7), 0, {}),
    (W["tiny"].replace(B=1), 0, {}),                                      # fewer rows than the call before
    (W["tiers_64k"].replace(B=2, ctx=16 * 300), 3, {"n_force_first": 1, "n_force_last": 2}),
    (W["qwen3b_128k"].replace(B=1, ctx=16 * 200 + 9), 0, {"coverage": 0.8}),
]


def test_noalloc_step_equals_workspace_step(hz, kv):
    for w, splits, sel in CASES:
        lens = [w.ctx] + [max(1, w.ctx - (5 + 3 * i) * w.P - 3) for i in range(1, w.B)]
        announce(f"no-alloc step {w.name} B={w.B} ctx={w.ctx} splits={splits} {sel} seq_lens={lens}")
        layer = hz.DeviceLayer(w, summaries="synthetic", seq_lens=lens)
        q = hz.queries_device(w)
        cap = w.Np if "coverage" in sel else None
        ref = _fresh(hz, w, splits)
        got = _fresh(hz, w, splits)
        if cap:
            for f in (ref, got):
                f.sel = torch.full((w.B, w.Hkv, cap), -7, dtype=torch.int32, device="cuda")
            ref.ws = torch.zeros(max(1, kv.attn_workspace_size(layer.L, w.B, cap, splits) // 4),
                                 dtype=torch.float32, device="cuda")
        hz.whole_step(layer, q, ref, **sel)
        _noalloc(kv, layer, q, got, **sel)
        torch.cuda.synchronize()
        for a, b in zip(_outputs(ref), _outputs(got)):
            np.testing.assert_array_equal(b, a)
        assert int(got.sel_count.cpu().numpy().min()) >= 1


def test_noalloc_step_in_a_graph(hz, kv):
    w = W["llama8b_32k"].replace(B=2, ctx=16 * 257 + 1)
    announce("no-alloc step captured in a HIP graph")
    layer = hz.DeviceLayer(w, summaries="synthetic")
    qs = [hz.queries_device(w, qidx=i) for i in range(3)]
    qbuf = qs[0].clone()
    got = _fresh(hz, w, 0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _noalloc(kv, layer, qbuf, got)              # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _noalloc(kv, layer, qbuf, got)
    torch.cuda.synchronize()
    for i in (1, 2, 0, 1):
        qbuf.copy_(qs[i])
        ref = _fresh(hz, w, 0)
        hz.whole_step(layer, qs[i], ref)           # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for a, b in zip(_outputs(ref), _outputs(got)):
            np.testing.assert_array_equal(b, a)


def test_noalloc_rejects_oversized_calls(kv):
    """More partials than the library's array holds: KV_ERR_WORKSPACE, nothing launched."""
    import ctypes
    L = kv.layout(32, 8, 128, 16, 4, "bf16")
    pg = kv.KvPages()
    pg.k16 = pg.v16 = 0x10000
    fake = 0x10000
    # 64 rows x 256 splits x 4 heads x 130 floats = 34 MB > 33292288 bytes
    rc = kv.lib().kv_sparse_decode_step_noalloc(ctypes.byref(L), fake, fake, fake, ctypes.byref(pg), fake, fake, 8,
                                                2048, 0.08, 0, -1.0, 0, 0, fake, fake, fake, fake, 164, None, 256,
                                                fake, fake, None)
    assert rc == kv.KV_ERR_WORKSPACE
    rc = kv.lib().kv_sparse_decode_step_noalloc(ctypes.byref(L), fake, fake, fake, ctypes.byref(pg), fake, fake, 8,
                                                2048, 0.08, 0, -1.0, 0, 0, fake, fake, fake, fake, 163, None, 0,
                                                fake, fake, None)
    assert rc == kv.KV_ERR_INVALID_ARG
