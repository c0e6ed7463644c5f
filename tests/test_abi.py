"""The C-ABI library loads, exports every declared symbol, and rejects bad host
arguments with the documented status before any HIP call (CPU only: no call
here reaches a kernel launch)."""

import ctypes
import os
import re

import pytest

from quantized_kv_cache_summary_amd import kvsparse as kv

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "kvsparse.h")

pytestmark = pytest.mark.skipif(not os.path.exists(kv.LIB_PATH), reason="libkvsparse.so not built")


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return set(re.findall(r"\b(kv_[a-z0-9_]+)\s*\(", text)) - {"kv_layout", "kv_pages"}


def test_header_and_binding_agree():
    assert _declared() == set(kv.SYMBOLS)


def test_library_exports_every_declared_symbol():
    lib = ctypes.CDLL(kv.LIB_PATH)
    for name in _declared():
        assert hasattr(lib, name), name


def test_status_strings():
    assert kv.status_string(0) == "ok"
    for s in (-1, -2, -3, -4):
        assert kv.status_string(s) not in ("ok", "unknown status")
    assert kv.status_string(17) == "unknown status"


def _L(**kw):
    a = dict(num_q_heads=32, num_kv_heads=8, head_dim=128, page_size=16, rank=4, dtype="bf16")
    a.update(kw)
    return kv.layout(**a)


FAKE = 0x10000   # a 16-byte aligned non-null address; never dereferenced (validation fails first)


def _score(L, **over):
    a = dict(q=FAKE, summary=FAKE, log_n=FAKE, sl=FAKE, B=2, max_pages=10, hs=FAKE, lp=FAKE)
    a.update(over)
    return kv.lib().kv_page_score(ctypes.byref(L), a["q"], a["summary"], a["log_n"], a["sl"],
                                  a["B"], a["max_pages"], a["hs"], a["lp"], None)


def test_layout_validation():
    assert _score(_L(head_dim=96)) == kv.KV_ERR_UNSUPPORTED
    assert _score(_L(page_size=8)) == kv.KV_ERR_UNSUPPORTED
    assert _score(_L(rank=3)) == kv.KV_ERR_UNSUPPORTED
    assert _score(_L(num_q_heads=12, num_kv_heads=8)) == kv.KV_ERR_INVALID_ARG
    assert _score(_L(num_q_heads=34, num_kv_heads=2)) == kv.KV_ERR_UNSUPPORTED   # G = 17
    assert _score(_L(num_kv_heads=0)) == kv.KV_ERR_INVALID_ARG
    L = _L()
    L.kv_dtype = 7
    assert _score(L) == kv.KV_ERR_UNSUPPORTED
    assert kv.lib().kv_page_score(None, FAKE, FAKE, FAKE, FAKE, 1, 1, FAKE, FAKE, None) == kv.KV_ERR_INVALID_ARG


def test_score_argument_validation():
    L = _L()
    assert _score(L, q=None) == kv.KV_ERR_INVALID_ARG
    assert _score(L, lp=None) == kv.KV_ERR_INVALID_ARG
    assert _score(L, summary=FAKE + 4) == kv.KV_ERR_INVALID_ARG    # misaligned
    assert _score(L, q=FAKE + 2) == kv.KV_ERR_INVALID_ARG          # misaligned
    assert _score(L, B=-1) == kv.KV_ERR_INVALID_ARG
    assert _score(L, B=0) == kv.KV_OK                              # nothing to do, no launch


def test_topk_validation():
    L = _L()
    f = kv.lib().kv_page_topk
    ok = dict(hs=FAKE, lp=FAKE, sl=FAKE, B=2, mp=100, keep=0.08, kf=0, ff=0, fl=0, sel=FAKE, cnt=FAKE,
              kmax=8, S=None)

    def call(**o):
        a = dict(ok)
        a.update(o)
        return f(ctypes.byref(L), a["hs"], a["lp"], a["sl"], a["B"], a["mp"], a["keep"], a["kf"], a["ff"],
                 a["fl"], a["sel"], a["cnt"], a["kmax"], a["S"], None, 0, None)

    assert call(kmax=7) == kv.KV_ERR_INVALID_ARG                   # ceil(0.08 * 100) = 8 > 7
    assert call(kf=20, kmax=19) == kv.KV_ERR_INVALID_ARG
    assert call(keep=float("nan")) == kv.KV_ERR_INVALID_ARG
    assert call(keep=-0.5) == kv.KV_ERR_INVALID_ARG
    assert call(mp=20000, kmax=2000) == kv.KV_ERR_UNSUPPORTED
    assert call(sel=None) == kv.KV_ERR_INVALID_ARG
    assert call(ff=-1) == kv.KV_ERR_INVALID_ARG
    assert call(B=0) == kv.KV_OK


def test_attention_validation_and_workspace():
    L = _L()
    pg = kv.KvPages()
    pg.k16 = FAKE
    pg.v16 = FAKE
    f = kv.lib().kv_sparse_decode_attn

    def call(pages=pg, ws=FAKE, ws_bytes=1 << 40, splits=0, q=FAKE):
        return f(ctypes.byref(L), q, ctypes.byref(pages) if pages is not None else None, FAKE, FAKE, 8, 2048,
                 FAKE, FAKE, 164, splits, FAKE, FAKE, ws, ws_bytes, None)

    s = kv.attn_num_splits(L, 8, 164)                  # native pages: one block per CU
    st = kv.attn_num_splits(L, 8, 164, tiered=True)    # packed tiers: two blocks per CU
    assert (s, st) == (4, 8)
    assert kv.attn_num_splits(L, 8, 16) == 2           # at least two pages per wave
    need = kv.attn_workspace_size(L, 8, 164, s)
    assert need == 64 * s * 4 * 130 * 4 + 64 * 4       # partials + one counter per row
    assert kv.attn_workspace_size(L, 8, 164) == kv.attn_workspace_size(L, 8, 164, st)
    assert call(ws_bytes=need - 1) == kv.KV_ERR_WORKSPACE
    assert call(ws=None) == kv.KV_ERR_WORKSPACE
    assert call(pages=None) == kv.KV_ERR_INVALID_ARG
    assert call(splits=300) == kv.KV_ERR_UNSUPPORTED
    assert call(q=FAKE + 8) == kv.KV_ERR_INVALID_ARG
    tiered = kv.KvPages()
    tiered.k16 = FAKE
    tiered.v16 = FAKE
    tiered.page_entry = FAKE
    assert call(pages=tiered) == kv.KV_ERR_INVALID_ARG              # tier pools missing
    hot = kv.KvPages()
    hot.k16 = FAKE
    hot.v16 = FAKE
    hot.v_hot_slot = FAKE
    assert call(pages=hot) == kv.KV_ERR_INVALID_ARG                 # hot buffer missing
    kh = kv.KvPages()
    kh.k16 = FAKE
    kh.v16 = FAKE
    kh.k_hot = FAKE
    assert call(pages=kh) == kv.KV_ERR_INVALID_ARG                  # K hot buffer without the slot map
    ko = kv.KvPages()
    ko.k16 = FAKE
    ko.v16 = FAKE
    ko.page_entry = FAKE
    for t in range(kv.NUM_PACKED_TIERS):
        ko.kq[t] = ko.vq[t] = ko.ksz[t] = ko.vsz[t] = FAKE
    ko.kout = FAKE
    assert call(pages=ko) == kv.KV_ERR_INVALID_ARG                  # K outlier table without V's


def test_fused_topk_attention_validation():
    L = _L()
    pg = kv.KvPages()
    pg.k16 = FAKE
    pg.v16 = FAKE
    f = kv.lib().kv_topk_sparse_decode_attn
    s = kv.attn_num_splits(L, 8, 164)
    need = kv.attn_workspace_size(L, 8, 164, s)

    def call(L=L, pages=pg, max_pages=2048, keep=0.08, k_fixed=0, coverage=-1.0, k_max=164, sel=FAKE,
             hs=FAKE, splits=0, ws=FAKE, ws_bytes=need, q=FAKE):
        return f(ctypes.byref(L), q, ctypes.byref(pages) if pages is not None else None, FAKE, FAKE, 8,
                 max_pages, hs, FAKE, keep, k_fixed, coverage, 0, 0, sel, FAKE, k_max, None, splits, FAKE,
                 FAKE, ws, ws_bytes, None)

    assert call(ws_bytes=need - 1) == kv.KV_ERR_WORKSPACE
    assert call(ws=None) == kv.KV_ERR_WORKSPACE
    assert call(k_max=163) == kv.KV_ERR_INVALID_ARG                 # ceil(0.08 * 2048) = 164
    assert call(keep=float("nan")) == kv.KV_ERR_INVALID_ARG
    assert call(coverage=float("nan")) == kv.KV_ERR_INVALID_ARG
    assert call(coverage=float("inf")) == kv.KV_ERR_INVALID_ARG
    assert call(coverage=0.9, k_max=0, sel=None) == kv.KV_ERR_INVALID_ARG
    assert call(sel=None) == kv.KV_ERR_INVALID_ARG
    assert call(hs=None) == kv.KV_ERR_INVALID_ARG
    assert call(pages=None) == kv.KV_ERR_INVALID_ARG
    assert call(q=FAKE + 8) == kv.KV_ERR_INVALID_ARG
    assert call(splits=300) == kv.KV_ERR_UNSUPPORTED
    assert call(max_pages=15361, k_max=15361) == kv.KV_ERR_UNSUPPORTED
    # the row's keys and a split's share of the selection must fit one block's LDS
    assert kv.topk_attn_supported(L, 2048, 164, s)
    assert kv.topk_attn_supported(_L(num_q_heads=64), 2048, 2048, 1)        # G = 8, the widest group
    assert not kv.topk_attn_supported(_L(num_q_heads=128), 2048, 2048, 1)   # G = 16: refused
    assert not kv.topk_attn_supported(L, 15360, 15360, 1)
    assert call(max_pages=15360, k_max=15360, keep=1.0, splits=1,
                ws_bytes=kv.attn_workspace_size(L, 8, 15360, 1)) == kv.KV_ERR_UNSUPPORTED
    assert not kv.topk_attn_supported(L, 2048, 164, 0)


def test_decode_step_validation():
    L = _L()
    pg = kv.KvPages()
    pg.k16 = FAKE
    pg.v16 = FAKE
    f = kv.lib().kv_sparse_decode_step
    s = kv.attn_num_splits(L, 8, 164)
    need = kv.step_workspace_size(L, 8, 164)
    assert need == kv.attn_workspace_size(L, 8, 164, 0)
    assert kv.step_workspace_size(L, 0, 164) == 0

    def call(L=L, pages=pg, B=8, max_pages=2048, keep=0.08, k_fixed=0, coverage=-1.0, k_max=164, sel=FAKE,
             summary=FAKE, splits=0, ws=FAKE, ws_bytes=need, q=FAKE, hs=FAKE):
        return f(ctypes.byref(L), q, summary, FAKE, ctypes.byref(pages) if pages is not None else None, FAKE,
                 FAKE, B, max_pages, keep, k_fixed, coverage, 0, 0, hs, FAKE, sel, FAKE, k_max, None, splits,
                 FAKE, FAKE, ws, ws_bytes, None)

    assert call(B=0) == kv.KV_OK
    assert call(ws_bytes=kv.attn_workspace_size(L, 8, 164, s) - 1) == kv.KV_ERR_WORKSPACE
    assert call(ws=None) == kv.KV_ERR_WORKSPACE
    assert call(max_pages=0) == kv.KV_ERR_INVALID_ARG
    assert call(k_max=163) == kv.KV_ERR_INVALID_ARG                 # ceil(0.08 * 2048) = 164
    assert call(keep=float("nan")) == kv.KV_ERR_INVALID_ARG
    assert call(coverage=float("inf")) == kv.KV_ERR_INVALID_ARG
    assert call(sel=None) == kv.KV_ERR_INVALID_ARG
    assert call(summary=None) == kv.KV_ERR_INVALID_ARG
    assert call(hs=None) == kv.KV_ERR_INVALID_ARG
    assert call(summary=FAKE + 8) == kv.KV_ERR_INVALID_ARG
    assert call(pages=None) == kv.KV_ERR_INVALID_ARG
    assert call(splits=300) == kv.KV_ERR_UNSUPPORTED
    assert call(max_pages=15361, k_max=15361) == kv.KV_ERR_UNSUPPORTED
    assert kv.step_supported(L, 8, 2048, 164)
    assert kv.step_supported(_L(num_q_heads=64), 8, 8192, 410)
    assert not kv.step_supported(L, 8, 15361, 15361, 1)
    assert not kv.step_supported(L, 8, 0, 1)
    # the fused launch where it measured faster: native pages, G <= 4, rows under 4096 pages
    assert kv.step_fused(L, pg, 8, 2048, 164)
    assert not kv.step_fused(L, pg, 8, 4096, 410)
    assert not kv.step_fused(_L(num_q_heads=64), pg, 8, 2048, 164)
    tiered = kv.KvPages()
    tiered.k16 = tiered.v16 = tiered.page_entry = FAKE
    for t in range(kv.NUM_PACKED_TIERS):
        tiered.kq[t] = tiered.vq[t] = tiered.ksz[t] = tiered.vsz[t] = FAKE
    assert not kv.step_fused(L, tiered, 4, 4096, 410)


def test_pack_build_dequant_validation():
    L = _L()
    lib = kv.lib()
    pt = lib.kv_pack_tier
    assert pt(ctypes.byref(L), FAKE, None, 4, 0, FAKE, FAKE, None, None, None) == kv.KV_ERR_UNSUPPORTED
    assert pt(ctypes.byref(L), FAKE, None, 4, 6, FAKE, FAKE, None, None, None) == kv.KV_ERR_UNSUPPORTED
    assert pt(ctypes.byref(L), FAKE, None, 0, kv.KV_TIER_FP8, FAKE, FAKE, None, None, None) == kv.KV_OK
    assert pt(ctypes.byref(L), None, None, 4, 1, FAKE, FAKE, None, None, None) == kv.KV_ERR_INVALID_ARG
    assert pt(ctypes.byref(L), FAKE, None, 0, 1, FAKE, FAKE, None, None, None) == kv.KV_OK
    assert pt(ctypes.byref(L), FAKE, None, 4, kv.KV_TIER_I8, FAKE, FAKE, FAKE, None, None) == kv.KV_ERR_INVALID_ARG
    sb = lib.kv_summary_build
    assert sb(ctypes.byref(L), FAKE, FAKE, 8, FAKE, FAKE, -1, FAKE, FAKE, None) == kv.KV_ERR_INVALID_ARG
    assert sb(ctypes.byref(L), FAKE + 4, FAKE, 8, FAKE, FAKE, 3, FAKE, FAKE, None) == kv.KV_ERR_INVALID_ARG
    assert sb(ctypes.byref(L), FAKE, None, 8, FAKE, FAKE, 3, FAKE, FAKE, None) == kv.KV_ERR_INVALID_ARG
    assert sb(ctypes.byref(L), FAKE, FAKE, 0, FAKE, FAKE, 3, FAKE, FAKE, None) == kv.KV_ERR_INVALID_ARG
    assert sb(ctypes.byref(L), FAKE, FAKE, 8, FAKE, FAKE, 0, FAKE, FAKE, None) == kv.KV_OK
    assert lib.kv_dequant_tier(ctypes.byref(L), None, FAKE, 2, FAKE, None) == kv.KV_ERR_INVALID_ARG
    assert kv.page_score_partial_size(L, 8, 2048) == 64 * 32 * 4 * 2 * 4
    assert kv.page_topk_workspace_size(L, 8, 2048) == 0


def test_shared_basis_validation():
    L = _L()
    lib = kv.lib()
    need = kv.basis_build_workspace_size(L, 2, 300)
    assert need == 16 * 2 * (1 + 128 + 128 * 128) * 4           # rows x 256-page chunks x statistics
    bb = lambda **o: lib.kv_basis_build(ctypes.byref(L), o.get("k", FAKE), FAKE, FAKE, 2, 300,
                                        o.get("basis", FAKE), None, o.get("ws", FAKE), o.get("wsb", need), None)
    assert bb(wsb=need - 1) == kv.KV_ERR_WORKSPACE
    assert bb(ws=None) == kv.KV_ERR_WORKSPACE
    assert bb(basis=None) == kv.KV_ERR_INVALID_ARG
    assert bb(k=FAKE + 2) == kv.KV_ERR_INVALID_ARG
    assert lib.kv_basis_build(ctypes.byref(L), FAKE, FAKE, FAKE, 0, 300, FAKE, None, None, 0, None) == kv.KV_OK
    sb = lambda **o: lib.kv_summary_build_basis(ctypes.byref(L), FAKE, FAKE, 300, FAKE, FAKE, o.get("n", 4),
                                                o.get("basis", FAKE), o.get("mu", FAKE), FAKE, FAKE, None)
    assert sb(basis=None) == kv.KV_ERR_INVALID_ARG
    assert sb(mu=None) == kv.KV_ERR_INVALID_ARG
    assert sb(n=-1) == kv.KV_ERR_INVALID_ARG
    assert sb(n=0) == kv.KV_OK
    ps = lambda **o: lib.kv_page_score_basis(ctypes.byref(L), FAKE, o.get("mu", FAKE), o.get("lam", FAKE),
                                             o.get("basis", FAKE), FAKE, FAKE, 2, 300, FAKE, FAKE, None)
    assert ps(mu=FAKE + 4) == kv.KV_ERR_INVALID_ARG
    assert ps(basis=FAKE + 4) == kv.KV_ERR_INVALID_ARG
    assert ps(lam=FAKE + 2) == kv.KV_ERR_INVALID_ARG
    assert ps(lam=None) == kv.KV_ERR_INVALID_ARG
    assert _score(_L(head_dim=96)) == kv.KV_ERR_UNSUPPORTED


def test_hot_admit_validation_and_workspace():
    L = _L()
    f = kv.lib().kv_hot_admit
    # count + 100 (unit, slot) pairs + 100 misses = 301 words, padded to 320; the
    # bitmap of 1000 units (32 words) ends at 352, padded to 384; 100 slot keys end
    # at 484, padded to 512; one word block's miss count ends at 513, padded to
    # 576; one slot block's two victim counts end at 578, padded to 640; 4 scalars
    assert kv.hot_admit_workspace_size(100, 1000) == 644 * 4
    assert kv.hot_admit_workspace_size(0, 1000) == 0
    assert kv.hot_admit_workspace_size(100, 0) == 0
    assert kv.hot_admit_workspace_size((1 << 22) + 1, 1000) == 0

    def call(v16=FAKE, v_hot=FAKE, k16=None, k_hot=None, hot=FAKE, n_units=1000, n_slots=100, step=1,
             ws=FAKE, ws_bytes=1 << 20, sel=FAKE, B=2):
        return f(ctypes.byref(L), v16, v_hot, k16, k_hot, hot, n_units, FAKE, FAKE, n_slots, FAKE, FAKE, B, 64,
                 sel, FAKE, 12, step, ws, ws_bytes, None)

    assert L.num_kv_heads == 8
    assert call(step=0) == kv.KV_ERR_INVALID_ARG                     # steps start at 1
    assert call(n_slots=0) == kv.KV_ERR_INVALID_ARG
    assert call(n_units=1004) == kv.KV_ERR_INVALID_ARG               # not n_phys * Hkv
    assert call(n_slots=(1 << 22) + 1) == kv.KV_ERR_UNSUPPORTED
    assert call(n_units=(1 << 24) + 8) == kv.KV_ERR_UNSUPPORTED
    assert call(v16=None) == kv.KV_ERR_INVALID_ARG
    assert call(v_hot=FAKE + 8) == kv.KV_ERR_INVALID_ARG
    assert call(hot=None) == kv.KV_ERR_INVALID_ARG
    assert call(k16=FAKE) == kv.KV_ERR_INVALID_ARG                   # K pool without a K hot buffer
    assert call(k_hot=FAKE) == kv.KV_ERR_INVALID_ARG                 # and the reverse
    assert call(sel=None) == kv.KV_ERR_INVALID_ARG
    assert call(ws_bytes=644 * 4 - 1) == kv.KV_ERR_WORKSPACE
    assert call(ws=None) == kv.KV_ERR_WORKSPACE
    assert call(ws=FAKE + 2) == kv.KV_ERR_WORKSPACE                  # not 4-byte aligned


def test_tier_plan_and_demote_validation():
    L = _L()
    lib = kv.lib()
    ok = (ctypes.c_int32 * 5)(1, 1, 1, 1, 1)
    bad = (ctypes.c_int32 * 5)(1, -1, 1, 1, 1)

    def plan(caps=ok, B=2, mp=64, S=FAKE, ff=0):
        return lib.kv_tier_plan(ctypes.byref(L), S, FAKE, B, mp, FAKE, FAKE, caps, ff, 0, FAKE, FAKE, None)

    assert plan(caps=None) == kv.KV_ERR_INVALID_ARG
    assert plan(caps=bad) == kv.KV_ERR_INVALID_ARG
    assert plan(ff=-1) == kv.KV_ERR_INVALID_ARG
    assert plan(mp=20000) == kv.KV_ERR_UNSUPPORTED
    assert plan(S=None) == kv.KV_ERR_INVALID_ARG
    assert plan(B=0) == kv.KV_OK
    pg = kv.KvPages()
    pg.k16 = FAKE
    pg.v16 = FAKE
    pg.page_entry = FAKE
    for t in range(kv.NUM_PACKED_TIERS):
        pg.kq[t] = pg.vq[t] = pg.ksz[t] = pg.vsz[t] = FAKE

    def demote(entry=FAKE, pages=pg, B=2):
        return lib.kv_tier_demote(ctypes.byref(L), ctypes.byref(pages) if pages is not None else None, entry, B, 64,
                                  FAKE, FAKE, None)

    assert demote(entry=FAKE + 16) == kv.KV_ERR_INVALID_ARG        # not the pools' own page_entry
    assert demote(pages=None) == kv.KV_ERR_INVALID_ARG
    assert demote(B=0) == kv.KV_OK
    pg.kq[2] = None
    assert demote() == kv.KV_ERR_INVALID_ARG                        # a tier pool missing


def test_lowrank_validation():
    L = _L(rank=8)
    lib = kv.lib()
    co = lambda **o: lib.kv_lowrank_coords(ctypes.byref(L), o.get("k", FAKE), FAKE, 300, FAKE, FAKE, o.get("n", 4),
                                           o.get("basis", FAKE), o.get("mean", FAKE), o.get("coords", FAKE), None)
    assert co(n=-1) == kv.KV_ERR_INVALID_ARG
    assert co(n=0) == kv.KV_OK
    assert co(mean=None) == kv.KV_ERR_INVALID_ARG
    assert co(coords=None) == kv.KV_ERR_INVALID_ARG
    assert co(k=FAKE + 2) == kv.KV_ERR_INVALID_ARG
    sc = lambda **o: lib.kv_page_score_lowrank(ctypes.byref(L), o.get("q", FAKE), o.get("coords", FAKE),
                                               FAKE, FAKE, FAKE, o.get("B", 2), 300, FAKE, FAKE, None)
    assert sc(coords=FAKE + 8) == kv.KV_ERR_INVALID_ARG
    assert sc(q=None) == kv.KV_ERR_INVALID_ARG
    assert sc(B=0) == kv.KV_OK
    assert lib.kv_page_score_lowrank(ctypes.byref(_L(rank=3)), FAKE, FAKE, FAKE, FAKE, FAKE, 2, 300, FAKE, FAKE,
                                     None) == kv.KV_ERR_UNSUPPORTED


def test_attention_refuses_groups_wider_than_eight():
    """Score and selection take up to 16 query heads per KV head; every call
    that runs the attention refuses more than 8 before any HIP call."""
    L16 = _L(num_q_heads=128)                       # G = 16
    pg = kv.KvPages()
    pg.k16 = pg.v16 = FAKE
    ws = kv.attn_workspace_size(L16, 8, 164)
    rc = kv.lib().kv_sparse_decode_attn(ctypes.byref(L16), FAKE, ctypes.byref(pg), FAKE, FAKE, 8, 2048, FAKE, FAKE,
                                        164, 0, FAKE, FAKE, FAKE, ws, None)
    assert rc == kv.KV_ERR_UNSUPPORTED
    rc = kv.lib().kv_topk_sparse_decode_attn(ctypes.byref(L16), FAKE, ctypes.byref(pg), FAKE, FAKE, 8, 2048, FAKE,
                                             FAKE, 0.08, 0, -1.0, 0, 0, FAKE, FAKE, 164, None, 0, FAKE, FAKE, FAKE,
                                             ws, None)
    assert rc == kv.KV_ERR_UNSUPPORTED
    rc = kv.lib().kv_sparse_decode_step(ctypes.byref(L16), FAKE, FAKE, FAKE, ctypes.byref(pg), FAKE, FAKE, 8, 2048,
                                        0.08, 0, -1.0, 0, 0, FAKE, FAKE, FAKE, FAKE, 164, None, 0, FAKE, FAKE, FAKE,
                                        ws, None)
    assert rc == kv.KV_ERR_UNSUPPORTED
    assert not kv.step_supported(L16, 8, 2048, 164)
    assert not kv.topk_attn_supported(L16, 2048, 164, 4)
    assert kv.step_supported(_L(num_q_heads=64), 8, 2048, 164)        # G = 8


def test_noalloc_step_validation():
    """The whole step without a workspace: the same argument rules as the
    workspace call, and calls whose partials exceed the library's array are
    refused with KV_ERR_WORKSPACE, all before any HIP call."""
    L = _L()
    pg = kv.KvPages()
    pg.k16 = pg.v16 = FAKE
    f = kv.lib().kv_sparse_decode_step_noalloc

    def call(L=L, B=8, max_pages=2048, k_max=164, splits=0, sel=FAKE, summary=FAKE):
        return f(ctypes.byref(L), FAKE, summary, FAKE, ctypes.byref(pg), FAKE, FAKE, B, max_pages, 0.08, 0, -1.0,
                 0, 0, FAKE, FAKE, sel, FAKE, k_max, None, splits, FAKE, FAKE, None)

    assert call(B=0) == kv.KV_OK
    assert call(k_max=163) == kv.KV_ERR_INVALID_ARG
    assert call(sel=None) == kv.KV_ERR_INVALID_ARG
    assert call(summary=FAKE + 8) == kv.KV_ERR_INVALID_ARG
    assert call(splits=300) == kv.KV_ERR_UNSUPPORTED
    assert call(L=_L(num_q_heads=128)) == kv.KV_ERR_UNSUPPORTED                  # G = 16
    # 64 rows x 256 splits x 4 heads x 130 floats = 34 MB: more than the 33292288 bytes of partials
    assert call(splits=256) == kv.KV_ERR_WORKSPACE
