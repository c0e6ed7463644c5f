"""GPU parity of hot-buffer admission (kv_hot_admit) against the oracle's rule.

The buffer's unit is one (physical page, KV head), u = phys * Hkv + g.  Over a
sequence of steps with seeded selections, after every step the three state
arrays (unit -> slot, slot -> unit, slot stamps) and the copy list must equal
the oracle's exactly, and every hot slot must hold its unit's V bit for bit.
With the V pool in pinned, device-mapped host memory, attention results must
not depend on which units are hot (the same bits are read from either place),
and the standalone decode reads every page's K and V through the buffer.
"""

import numpy as np
import pytest
import torch

import oracle
from quantized_kv_cache_summary_amd import workloads as wl

pytestmark = pytest.mark.gpu

W = wl.WORKLOADS


def announce(msg):
    print(f"[case] {msg}", flush=True)


@pytest.fixture(scope="module")
def hz():
    from quantized_kv_cache_summary_amd import harness
    return harness


def _step_selection(w, rng, k_max, lens):
    """A step's selection: per row a random count in [0, k_max] of sorted distinct pages
    (some past the row's length, some -1 padding), as the top-k would leave it."""
    sel = np.full((w.B, w.Hkv, k_max), -1, dtype=np.int32)
    cnt = np.zeros((w.B, w.Hkv), dtype=np.int32)
    for b in range(w.B):
        for g in range(w.Hkv):
            k = int(rng.integers(0, k_max + 1))
            pick = np.sort(rng.choice(w.Np, size=min(k, w.Np), replace=False))
            sel[b, g, :pick.size] = pick
            cnt[b, g] = pick.size + (1 if rng.random() < 0.1 else 0)   # a count past the list
    return sel, cnt


@pytest.mark.parametrize("name,n_slots", [("llama_small", 40), ("heavy_small", 13), ("heavy_small", 400),
                                          ("llama_small", 40000)])
def test_admission_matches_oracle(hz, name, n_slots):
    from quantized_kv_cache_summary_amd import kvsparse as kv
    w = {"llama_small": W["llama8b_32k"].replace(B=2, ctx=16 * 300 + 7),
         "heavy_small": W["heavy70b_128k"].replace(B=2, Hq=16, Hkv=2, ctx=32 * 150 + 5, v_host=False)}[name]
    announce(f"hot admission {name} slots={n_slots}")
    lens = [w.ctx, w.ctx - 7 * w.P]
    layer = hz.DeviceLayer(w, summaries=None, seq_lens=lens)
    L = layer.L
    n_units = w.n_phys * w.Hkv
    hot = torch.full((n_units,), -1, dtype=torch.int32, device="cuda")
    slot_page = torch.full((n_slots,), -1, dtype=torch.int32, device="cuda")
    slot_stamp = torch.zeros((n_slots,), dtype=torch.int32, device="cuda")
    v_hot = torch.zeros((n_slots, w.P, w.d), dtype=layer.v16.dtype, device="cuda")
    ws = torch.full((kv.hot_admit_workspace_size(n_slots, n_units) // 4,), -7, dtype=torch.int32, device="cuda")
    ref = oracle.HotBuffer(n_units, n_slots)
    rng = np.random.default_rng(41 + n_slots)
    k_max = 12 if n_slots < 1000 else 160
    v_all = layer.v16.view(torch.int16).cpu().numpy().reshape(n_units, -1)
    for t in range(1, 16):
        sel, cnt = _step_selection(w, rng, k_max, lens)
        kv.hot_admit(L, layer.v16.data_ptr(), v_hot, hot, slot_page, slot_stamp, layer.bt, layer.seq_lens,
                     torch.from_numpy(sel).cuda(), torch.from_numpy(cnt).cuda(), t, ws)
        torch.cuda.synchronize()
        U = oracle.selected_units(sel, cnt, layer.bt_np, w.Hkv, np.array(lens), w.P)
        copies = ref.step(U, t)
        assert np.array_equal(hot.cpu().numpy(), ref.hot), t
        assert np.array_equal(slot_page.cpu().numpy(), ref.slot_page), t
        assert np.array_equal(slot_stamp.cpu().numpy().astype(np.int64), ref.slot_stamp), t
        wsn = ws.cpu().numpy()
        assert wsn[0] == len(copies) and [tuple(x) for x in wsn[1:1 + 2 * len(copies)].reshape(-1, 2)] == copies
        vh = v_hot.view(torch.int16).cpu().numpy().reshape(n_slots, -1)
        for s, u in enumerate(ref.slot_page):
            if u >= 0:
                assert np.array_equal(vh[s], v_all[u]), (t, s, u)


def test_admission_from_host_mapped_pool_keeps_attention(hz):
    from quantized_kv_cache_summary_amd import kvsparse as kv
    w = W["heavy70b_128k"].replace(B=2, Hq=16, Hkv=2, ctx=32 * 150 + 5)     # V in mapped host memory
    announce("hot admission from host-mapped V")
    layer = hz.DeviceLayer(w, summaries="build", hot_mode="cold")
    try:
        q = hz.queries_device(w)
        bufs = hz.StepBuffers(w)
        hz.score(layer, q, bufs)
        hz.topk(layer, bufs)
        hz.attend(layer, q, bufs)
        torch.cuda.synchronize()
        out0, lse0 = bufs.out.cpu().numpy().copy(), bufs.lse.cpu().numpy().copy()
        n_slots = layer.v_hot.shape[0]
        slot_page = torch.from_numpy(np.array(layer.hot_units, dtype=np.int32)).cuda()
        if slot_page.numel() < n_slots:
            slot_page = torch.cat([slot_page, torch.full((n_slots - slot_page.numel(),), -1, dtype=torch.int32,
                                                          device="cuda")])
        slot_stamp = torch.zeros(n_slots, dtype=torch.int32, device="cuda")
        hot = layer.v_hot_slot.clone()
        ws = torch.zeros(kv.hot_admit_workspace_size(n_slots, hot.shape[0]) // 4, dtype=torch.int32, device="cuda")
        kv.hot_admit(layer.L, layer.host_v.dev.value, layer.v_hot, hot, slot_page, slot_stamp, layer.bt,
                     layer.seq_lens, bufs.sel, bufs.sel_count, 1, ws)
        torch.cuda.synchronize()
        layer.v_hot_slot = hot
        layer.pages = layer._make_pages()
        # every selected unit is hot now (the step fits the buffer) ...
        sel, cnt = bufs.sel.cpu().numpy(), bufs.sel_count.cpu().numpy()
        U = oracle.selected_units(sel, cnt, layer.bt_np, w.Hkv, layer.seq_lens_np, w.P)
        if U.size <= n_slots:
            assert np.all(hot.cpu().numpy()[U] >= 0)
        # ... and attention reads the same bits from the buffer
        hz.attend(layer, q, bufs)
        torch.cuda.synchronize()
        np.testing.assert_array_equal(bufs.out.cpu().numpy(), out0)
        np.testing.assert_array_equal(bufs.lse.cpu().numpy(), lse0)
    finally:
        layer.release()


def test_mem_kv_pool_with_admission_matches_resident(hz):
    """K and V both in device-mapped host memory (mem-kv) with a hot buffer for
    each, driven step by step with admission before every attention: every
    step's selection and attention are bit-identical to the same layer held in
    HBM, and every hot slot holds its unit's K and V."""
    from parity import assert_attn_close, check_selection
    base = W["heavy70b_128k"].replace(B=2, Hq=16, Hkv=2, ctx=32 * 150 + 5)
    announce("mem-kv pool (K and V host-mapped) against the resident layer")
    res = hz.DeviceLayer(base.replace(v_host=False), summaries="build")
    mem = hz.DeviceLayer(base.replace(k_host=True), summaries="build", hot_mode="cold")
    try:
        assert mem.k16 is None and mem.k_hot is not None
        np.testing.assert_array_equal(mem.summary.view(torch.int16).cpu().numpy(),
                                      res.summary.view(torch.int16).cpu().numpy())
        rbufs = hz.StepBuffers(base)
        ms = hz.MemStep(mem)
        w = base
        for t in range(6):
            q = hz.queries_device(w, 0, t % 2)          # steps repeat, so later ones hit the buffer
            hz.decode_step(res, q, rbufs)
            mb = ms(q)
            torch.cuda.synchronize()
            np.testing.assert_array_equal(mb.sel_count.cpu().numpy(), rbufs.sel_count.cpu().numpy())
            np.testing.assert_array_equal(mb.sel.cpu().numpy(), rbufs.sel.cpu().numpy())
            np.testing.assert_array_equal(mb.out.cpu().numpy(), rbufs.out.cpu().numpy())
            np.testing.assert_array_equal(mb.lse.cpu().numpy(), rbufs.lse.cpu().numpy())
        # the buffer's contents follow its map, for K and V
        kh = mem.host_k.numpy(np.uint16, (w.n_phys * w.Hkv, w.P, w.d))
        vh = mem.host_v.numpy(np.uint16, (w.n_phys * w.Hkv, w.P, w.d))
        k_hot = mem.k_hot.view(torch.int16).cpu().numpy().view(np.uint16)
        v_hot = mem.v_hot.view(torch.int16).cpu().numpy().view(np.uint16)
        slot_page = ms.slot_page.cpu().numpy()
        hot = mem.v_hot_slot.cpu().numpy()
        assert (slot_page >= 0).sum() == k_hot.shape[0]
        for s, u in enumerate(slot_page):
            assert hot[u] == s
            np.testing.assert_array_equal(k_hot[s], kh[u])
            np.testing.assert_array_equal(v_hot[s], vh[u])
        # and the last step against the oracle on every row
        sel, out, lse = mb.sel.cpu().numpy(), mb.out.cpu().numpy(), mb.lse.cpu().numpy()
        for b in range(w.B):
            for g in range(w.Hkv):
                r = oracle.decode_row(wl.queries(w, 0, b, g, qidx=1).astype(np.float64),
                                      wl.row_keys(w, 0, b, g), wl.row_values(w, 0, b, g), w.ctx, w.P, w.rank,
                                      w.tau, w.keep, w.k_fixed)
                k = r["k"]
                check_selection(r["S"], k, sel[b, g, :k], rel=1e-3)
                if set(sel[b, g, :k].tolist()) == set(r["sel"].tolist()):
                    hs = slice(g * w.G, (g + 1) * w.G)
                    assert_attn_close(out[b, hs], lse[b, hs], r["out"], r["lse"])
    finally:
        mem.release()


@pytest.mark.parametrize("host_k", [False, True])
def test_dequant_reads_through_the_hot_buffer(hz, host_k):
    """kv_dequant_tier over a layer whose V (and, mem-kv, K) sit in device-mapped
    host memory behind a buffer of (page, KV head) units: every page's K and V
    come out equal to the pool's values, whichever of its units are hot."""
    from quantized_kv_cache_summary_amd import kvsparse as kv
    w = W["heavy70b_128k"].replace(B=2, Hq=16, Hkv=2, ctx=32 * 150 + 5, k_host=host_k)
    announce(f"dequant through the hot buffer, K in host memory: {host_k}")
    layer = hz.DeviceLayer(w, summaries=None, hot_mode="cold")
    try:
        ids_np = np.arange(w.n_phys, dtype=np.int32)
        out = torch.empty((w.n_phys, 2, w.Hkv, w.P, w.d), dtype=torch.float32, device="cuda")
        kv.dequant_tier(layer.L, layer.pages, torch.from_numpy(ids_np).cuda(), out)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        shape = (w.n_phys, w.Hkv, w.P, w.d)
        kpool = (layer.host_k.numpy(np.uint16, shape) if host_k
                 else layer.k16.view(torch.int16).cpu().numpy().view(np.uint16).reshape(shape))
        vpool = layer.host_v.numpy(np.uint16, shape)
        np.testing.assert_array_equal(out[:, 0], wl.bits_to_f32(kpool, w.dtype))
        np.testing.assert_array_equal(out[:, 1], wl.bits_to_f32(vpool, w.dtype))
        hot = layer.v_hot_slot.cpu().numpy()
        assert (hot >= 0).any() and (hot < 0).any()      # both kinds of unit were read
    finally:
        layer.release()


def test_tiered_layout_reads_native_values_through_the_hot_buffer(hz):
    """A tiered layout with a unit hot buffer: the native pages' values are read
    from the buffer where their unit is hot, and the attention is bit-identical
    to the same layout without a buffer (packed tiers keep their own pools)."""
    from quantized_kv_cache_summary_amd import kvsparse as kv
    w = W["tiers_64k"].replace(B=2, ctx=16 * 300 + 7)
    announce("tiered layout with a hot buffer of native units")
    layer = hz.DeviceLayer(w, summaries=None)
    q = hz.queries_device(w)
    sel_np, cnt_np = wl.synthetic_selection(w, w.k_of(w.Np), ragged=True)
    sel, cnt = torch.from_numpy(sel_np).cuda(), torch.from_numpy(cnt_np).cuda()
    bufs = hz.StepBuffers(w)
    hz.attend(layer, q, bufs, sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    out0, lse0 = bufs.out.cpu().numpy().copy(), bufs.lse.cpu().numpy().copy()
    n_units = w.n_phys * w.Hkv
    native_units = np.nonzero(np.repeat(layer.tier_phys == 0, w.Hkv))[0]
    units = native_units[::2]
    assert units.size > 0
    slot = np.full(n_units, -1, dtype=np.int32)
    slot[units] = np.arange(units.size, dtype=np.int32)
    # the buffer holds copies of the units' values; the pool keeps them too
    layer.v_hot = layer.v16.view(n_units, w.P, w.d)[torch.from_numpy(units).cuda()].contiguous()
    layer.v_hot_slot = torch.from_numpy(slot).cuda()
    layer.pages = layer._make_pages()
    bufs.out.fill_(float("nan"))
    hz.attend(layer, q, bufs, sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bufs.out.cpu().numpy(), out0)
    np.testing.assert_array_equal(bufs.lse.cpu().numpy(), lse0)
    # with the pool's values zeroed where the unit is hot, the result still holds
    # only because those units are read from the buffer
    pool = layer.v16.view(n_units, w.P, w.d)
    pool[torch.from_numpy(units).cuda()] = 0
    hz.attend(layer, q, bufs, sel=sel, sel_count=cnt)
    torch.cuda.synchronize()
    np.testing.assert_array_equal(bufs.out.cpu().numpy(), out0)
