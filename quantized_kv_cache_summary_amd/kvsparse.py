"""ctypes binding of libkvsparse (include/kvsparse.h).  Argument marshalling only.

Every function takes torch tensors for device buffers, passes their data
pointers, sizes and torch's current HIP stream to the C ABI, and raises
``KvError`` on a non-zero status.  The library is loaded on first use; if it has
not been built the call raises: there is no fallback path.
"""

from __future__ import annotations

import ctypes
import os

import torch

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libkvsparse.so")

KV_OK, KV_ERR_INVALID_ARG, KV_ERR_UNSUPPORTED, KV_ERR_WORKSPACE, KV_ERR_HIP = 0, -1, -2, -3, -4
KV_F16, KV_BF16 = 0, 1
KV_TIER_NATIVE, KV_TIER_I8, KV_TIER_I4, KV_TIER_I2, KV_TIER_B1, KV_TIER_FP8 = range(6)
NUM_PACKED_TIERS = 5
TIER_BITS = {KV_TIER_I8: 8, KV_TIER_I4: 4, KV_TIER_I2: 2, KV_TIER_B1: 1, KV_TIER_FP8: 8}

# every entry point declared in include/kvsparse.h
SYMBOLS = (
    "kv_summary_build", "kv_page_score", "kv_page_score_partial_size", "kv_page_topk",
    "kv_page_topk_workspace_size", "kv_sparse_decode_attn", "kv_sparse_decode_attn_workspace_size",
    "kv_sparse_decode_attn_num_splits", "kv_dequant_tier", "kv_pack_tier", "kv_status_string",
    "kv_basis_build", "kv_basis_build_workspace_size", "kv_summary_build_basis", "kv_page_score_basis",
    "kv_page_topk_coverage", "kv_hot_admit", "kv_hot_admit_workspace_size", "kv_tier_plan", "kv_tier_demote",
    "kv_lowrank_coords", "kv_page_score_lowrank", "kv_topk_sparse_decode_attn",
    "kv_topk_sparse_decode_attn_supported", "kv_sparse_decode_step", "kv_sparse_decode_step_workspace_size",
    "kv_sparse_decode_step_supported", "kv_sparse_decode_step_fused", "kv_sparse_decode_step_noalloc",
)


class KvError(RuntimeError):
    def __init__(self, status, fn):
        self.status = status
        super().__init__(f"{fn} failed: {status_string(status)} ({status})")


class KvLayout(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32), ("page_size", ctypes.c_int32), ("rank", ctypes.c_int32),
        ("kv_dtype", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
    ]


class KvPages(ctypes.Structure):
    _fields_ = [
        ("k16", ctypes.c_void_p), ("v16", ctypes.c_void_p),
        ("kq", ctypes.c_void_p * NUM_PACKED_TIERS), ("vq", ctypes.c_void_p * NUM_PACKED_TIERS),
        ("ksz", ctypes.c_void_p * NUM_PACKED_TIERS), ("vsz", ctypes.c_void_p * NUM_PACKED_TIERS),
        ("page_entry", ctypes.c_void_p), ("v_hot", ctypes.c_void_p), ("v_hot_slot", ctypes.c_void_p),
        ("k_hot", ctypes.c_void_p),
        ("kout", ctypes.c_void_p), ("vout", ctypes.c_void_p),
    ]


_lib = None
_P = ctypes.c_void_p
_I = ctypes.c_int32
_SZ = ctypes.c_size_t
_LP = ctypes.POINTER(KvLayout)
_PP = ctypes.POINTER(KvPages)


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built; run __graft_entry__.build() first")
        L = ctypes.CDLL(LIB_PATH)
        sig = {
            "kv_summary_build": (_I, [_LP, _P, _P, _I, _P, _P, _I, _P, _P, _P]),
            "kv_page_score": (_I, [_LP, _P, _P, _P, _P, _I, _I, _P, _P, _P]),
            "kv_page_score_partial_size": (_SZ, [_LP, _I, _I]),
            "kv_page_topk": (_I, [_LP, _P, _P, _P, _I, _I, ctypes.c_float, _I, _I, _I, _P, _P, _I, _P,
                                  _P, _SZ, _P]),
            "kv_page_topk_workspace_size": (_SZ, [_LP, _I, _I]),
            "kv_hot_admit": (_I, [_LP, _P, _P, _P, _P, _P, _I, _P, _P, _I, _P, _P, _I, _I, _P, _P, _I, ctypes.c_uint32,
                                  _P, _SZ, _P]),
            "kv_hot_admit_workspace_size": (_SZ, [_I, _I]),
            "kv_tier_plan": (_I, [_LP, _P, _P, _I, _I, _P, _P, ctypes.POINTER(ctypes.c_int32), _I, _I, _P, _P, _P]),
            "kv_tier_demote": (_I, [_LP, ctypes.POINTER(KvPages), _P, _I, _I, _P, _P, _P]),
            "kv_page_topk_coverage": (_I, [_LP, _P, _P, _P, _I, _I, ctypes.c_float, _I, _I, _P, _P, _I, _P,
                                           _P, _SZ, _P]),
            "kv_sparse_decode_attn": (_I, [_LP, _P, _PP, _P, _P, _I, _I, _P, _P, _I, _I, _P, _P, _P,
                                           _SZ, _P]),
            "kv_sparse_decode_attn_workspace_size": (_SZ, [_LP, _I, _I, _I]),
            "kv_topk_sparse_decode_attn": (_I, [_LP, _P, _PP, _P, _P, _I, _I, _P, _P, ctypes.c_float, _I,
                                                ctypes.c_float, _I, _I, _P, _P, _I, _P, _I, _P, _P, _P, _SZ,
                                                _P]),
            "kv_topk_sparse_decode_attn_supported": (_I, [_LP, _I, _I, _I]),
            "kv_sparse_decode_step": (_I, [_LP, _P, _P, _P, _PP, _P, _P, _I, _I, ctypes.c_float, _I,
                                           ctypes.c_float, _I, _I, _P, _P, _P, _P, _I, _P, _I, _P, _P, _P,
                                           _SZ, _P]),
            "kv_sparse_decode_step_noalloc": (_I, [_LP, _P, _P, _P, _PP, _P, _P, _I, _I, ctypes.c_float, _I,
                                                   ctypes.c_float, _I, _I, _P, _P, _P, _P, _I, _P, _I, _P, _P,
                                                   _P]),
            "kv_sparse_decode_step_workspace_size": (_SZ, [_LP, _I, _I, _I]),
            "kv_sparse_decode_step_supported": (_I, [_LP, _I, _I, _I, _I]),
            "kv_sparse_decode_step_fused": (_I, [_LP, _PP, _I, _I, _I, _I]),
            "kv_sparse_decode_attn_num_splits": (_I, [_LP, _I, _I, _I]),
            "kv_dequant_tier": (_I, [_LP, _PP, _P, _I, _P, _P]),
            "kv_pack_tier": (_I, [_LP, _P, _P, _I, _I, _P, _P, _P, _P, _P]),
            "kv_status_string": (ctypes.c_char_p, [ctypes.c_int]),
            "kv_basis_build": (_I, [_LP, _P, _P, _P, _I, _I, _P, _P, _P, _SZ, _P]),
            "kv_lowrank_coords": (_I, [_LP, _P, _P, _I, _P, _P, _I, _P, _P, _P, _P]),
            "kv_page_score_lowrank": (_I, [_LP, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P]),
            "kv_basis_build_workspace_size": (_SZ, [_LP, _I, _I]),
            "kv_summary_build_basis": (_I, [_LP, _P, _P, _I, _P, _P, _I, _P, _P, _P, _P, _P]),
            "kv_page_score_basis": (_I, [_LP, _P, _P, _P, _P, _P, _P, _I, _I, _P, _P, _P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def status_string(status):
    return lib().kv_status_string(int(status)).decode()


def layout(num_q_heads, num_kv_heads, head_dim, page_size, rank, dtype, softmax_scale=0.0):
    d = {"f16": KV_F16, "bf16": KV_BF16, torch.float16: KV_F16, torch.bfloat16: KV_BF16}[dtype]
    return KvLayout(num_q_heads, num_kv_heads, head_dim, page_size, rank, d, softmax_scale)


def _p(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return stream


def _check(rc, fn):
    if rc != KV_OK:
        raise KvError(rc, fn)


def make_pages(k16, v16, kq=None, vq=None, ksz=None, vsz=None, page_entry=None, v_hot=None,
               v_hot_slot=None, v16_ptr=None, k_hot=None, k16_ptr=None, kout=None, vout=None):
    """KvPages struct; keeps the tensors alive on the returned object.

    v16_ptr / k16_ptr override v16's / k16's pointer (a device-mapped host address)."""
    pg = KvPages()
    pg.k16 = k16_ptr if k16_ptr is not None else _p(k16)
    pg.v16 = v16_ptr if v16_ptr is not None else _p(v16)
    for t in range(NUM_PACKED_TIERS):
        pg.kq[t] = _p(kq[t]) if kq else None
        pg.vq[t] = _p(vq[t]) if vq else None
        pg.ksz[t] = _p(ksz[t]) if ksz else None
        pg.vsz[t] = _p(vsz[t]) if vsz else None
    pg.page_entry = _p(page_entry)
    pg.v_hot = _p(v_hot)
    pg.v_hot_slot = _p(v_hot_slot)
    pg.k_hot = _p(k_hot)
    pg.kout = _p(kout)
    pg.vout = _p(vout)
    pg._keep = (k16, v16, kq, vq, ksz, vsz, page_entry, v_hot, v_hot_slot, k_hot, kout, vout)
    return pg


def summary_build(L, k16, block_table, entries, n_valid, summary, log_n, stream=None):
    """entries: int32 (n, 2) of (sequence, logical page); summary [B, Hkv, max_pages, (1+R)*d]."""
    max_pages = block_table.shape[1]
    rc = lib().kv_summary_build(ctypes.byref(L), _p(k16), _p(block_table), int(max_pages), _p(entries),
                                _p(n_valid), int(entries.shape[0]), _p(summary), _p(log_n), _stream(stream))
    _check(rc, "kv_summary_build")


def basis_build_workspace_size(L, B, max_pages):
    return int(lib().kv_basis_build_workspace_size(ctypes.byref(L), int(B), int(max_pages)))


def basis_build(L, k16, block_table, seq_lens, basis, ws, stream=None, mean=None):
    B, max_pages = block_table.shape
    rc = lib().kv_basis_build(ctypes.byref(L), _p(k16), _p(block_table), _p(seq_lens), int(B), int(max_pages),
                              _p(basis), _p(mean), _p(ws), ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "kv_basis_build")


def summary_build_basis(L, k16, block_table, entries, n_valid, basis, mu, lam, log_n, stream=None):
    max_pages = block_table.shape[1]
    rc = lib().kv_summary_build_basis(ctypes.byref(L), _p(k16), _p(block_table), int(max_pages), _p(entries),
                                      _p(n_valid), int(n_valid.shape[0]), _p(basis), _p(mu), _p(lam),
                                      _p(log_n), _stream(stream))
    _check(rc, "kv_summary_build_basis")


def page_score_basis(L, q, mu, lam, basis, log_n, seq_lens, head_scores, lse_partial, stream=None):
    B = seq_lens.shape[0]
    max_pages = log_n.shape[1]
    rc = lib().kv_page_score_basis(ctypes.byref(L), _p(q), _p(mu), _p(lam), _p(basis), _p(log_n), _p(seq_lens),
                                   int(B), int(max_pages), _p(head_scores), _p(lse_partial), _stream(stream))
    _check(rc, "kv_page_score_basis")


def page_score_partial_size(L, B, max_pages):
    return int(lib().kv_page_score_partial_size(ctypes.byref(L), int(B), int(max_pages)))


def page_score(L, q, summary, log_n, seq_lens, head_scores, lse_partial, stream=None):
    """summary [B, Hkv, max_pages, (1+R)*d]; head_scores [B, Hkv, G, max_pages]."""
    B, max_pages = seq_lens.shape[0], summary.shape[2]
    rc = lib().kv_page_score(ctypes.byref(L), _p(q), _p(summary), _p(log_n), _p(seq_lens), int(B),
                             int(max_pages), _p(head_scores), _p(lse_partial), _stream(stream))
    _check(rc, "kv_page_score")


def page_topk_workspace_size(L, B, max_pages):
    return int(lib().kv_page_topk_workspace_size(ctypes.byref(L), int(B), int(max_pages)))


def page_topk(L, head_scores, lse_partial, seq_lens, max_pages, keep_frac, k_fixed, sel, sel_count,
              n_force_first=0, n_force_last=0, page_S=None, ws=None, stream=None):
    B = seq_lens.shape[0]
    k_max = sel.shape[-1]
    rc = lib().kv_page_topk(ctypes.byref(L), _p(head_scores), _p(lse_partial), _p(seq_lens), int(B),
                            int(max_pages), float(keep_frac), int(k_fixed), int(n_force_first),
                            int(n_force_last), _p(sel), _p(sel_count), int(k_max), _p(page_S), _p(ws),
                            0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "kv_page_topk")


def page_topk_coverage(L, head_scores, lse_partial, seq_lens, max_pages, coverage, sel, sel_count,
                       n_force_first=0, n_force_last=0, page_S=None, ws=None, stream=None):
    B = seq_lens.shape[0]
    k_max = sel.shape[-1]
    rc = lib().kv_page_topk_coverage(ctypes.byref(L), _p(head_scores), _p(lse_partial), _p(seq_lens), int(B),
                                     int(max_pages), float(coverage), int(n_force_first), int(n_force_last),
                                     _p(sel), _p(sel_count), int(k_max), _p(page_S), _p(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "kv_page_topk_coverage")


def hot_admit_workspace_size(n_slots, n_units):
    return int(lib().kv_hot_admit_workspace_size(int(n_slots), int(n_units)))


def hot_admit(L, v16_ptr, v_hot, v_hot_slot, slot_page, slot_stamp, block_table, seq_lens, sel, sel_count, step,
              ws, stream=None, k16_ptr=None, k_hot=None):
    """v16_ptr / k16_ptr: device addresses (int) of the V / K pools, which may be
    device-mapped host memory; K is admitted only with k16_ptr and k_hot.
    v_hot_slot: int32 [n_phys * Hkv], one entry per (physical page, KV head)."""
    B, max_pages = block_table.shape
    rc = lib().kv_hot_admit(ctypes.byref(L), ctypes.c_void_p(v16_ptr), _p(v_hot),
                            None if k16_ptr is None else ctypes.c_void_p(k16_ptr), _p(k_hot), _p(v_hot_slot),
                            int(v_hot_slot.shape[0]), _p(slot_page), _p(slot_stamp), int(slot_page.shape[0]),
                            _p(block_table), _p(seq_lens), int(B), int(max_pages), _p(sel), _p(sel_count),
                            int(sel.shape[-1]), int(step), _p(ws), ws.numel() * ws.element_size(),
                            _stream(stream))
    _check(rc, "kv_hot_admit")


def lowrank_coords(L, k16, block_table, entries, n_valid, basis, mean, coords, stream=None):
    max_pages = block_table.shape[1]
    rc = lib().kv_lowrank_coords(ctypes.byref(L), _p(k16), _p(block_table), int(max_pages), _p(entries),
                                 _p(n_valid), int(n_valid.numel()), _p(basis), _p(mean), _p(coords), _stream(stream))
    _check(rc, "kv_lowrank_coords")


def page_score_lowrank(L, q, coords, mean, basis, seq_lens, head_scores, lse_partial, stream=None):
    B, max_pages = head_scores.shape[0], head_scores.shape[-1]
    rc = lib().kv_page_score_lowrank(ctypes.byref(L), _p(q), _p(coords), _p(mean), _p(basis), _p(seq_lens),
                                     int(B), int(max_pages), _p(head_scores), _p(lse_partial), _stream(stream))
    _check(rc, "kv_page_score_lowrank")


def tier_plan(L, page_S, seq_lens, block_table, page_entry, caps, moves, move_count, n_force_first=0,
              n_force_last=0, stream=None):
    """caps: 5 page budgets (native, FP8, int8, int4, int2)."""
    B, max_pages = block_table.shape
    c = (ctypes.c_int32 * 5)(*[int(x) for x in caps])
    rc = lib().kv_tier_plan(ctypes.byref(L), _p(page_S), _p(seq_lens), int(B), int(max_pages), _p(block_table),
                            _p(page_entry), c, int(n_force_first), int(n_force_last), _p(moves), _p(move_count),
                            _stream(stream))
    _check(rc, "kv_tier_plan")


def tier_demote(L, pages, page_entry, block_table, moves, move_count, stream=None):
    B, max_pages = block_table.shape
    rc = lib().kv_tier_demote(ctypes.byref(L), ctypes.byref(pages), _p(page_entry), int(B), int(max_pages),
                              _p(moves), _p(move_count), _stream(stream))
    _check(rc, "kv_tier_demote")


def attn_num_splits(L, B, k_max, tiered=False):
    return int(lib().kv_sparse_decode_attn_num_splits(ctypes.byref(L), int(B), int(k_max), int(bool(tiered))))


def attn_workspace_size(L, B, k_max, num_splits=0):
    return int(lib().kv_sparse_decode_attn_workspace_size(ctypes.byref(L), int(B), int(k_max),
                                                          int(num_splits)))


def sparse_decode_attn(L, q, pages, block_table, seq_lens, sel, sel_count, out, lse, ws,
                       num_splits=0, stream=None):
    B, max_pages = block_table.shape
    k_max = sel.shape[-1]
    rc = lib().kv_sparse_decode_attn(ctypes.byref(L), _p(q), ctypes.byref(pages), _p(block_table),
                                     _p(seq_lens), int(B), int(max_pages), _p(sel), _p(sel_count),
                                     int(k_max), int(num_splits), _p(out), _p(lse), _p(ws),
                                     0 if ws is None else ws.numel() * ws.element_size(),
                                     _stream(stream))
    _check(rc, "kv_sparse_decode_attn")


def topk_attn_supported(L, max_pages, k_max, num_splits):
    return bool(lib().kv_topk_sparse_decode_attn_supported(ctypes.byref(L), int(max_pages), int(k_max),
                                                           int(num_splits)))


def topk_sparse_decode_attn(L, q, pages, block_table, seq_lens, head_scores, lse_partial, sel, sel_count,
                            out, lse, ws, keep_frac=0.0, k_fixed=0, coverage=-1.0, n_force_first=0,
                            n_force_last=0, page_S=None, num_splits=0, stream=None):
    """Selector and sparse attention in one launch; coverage < 0 selects by
    keep_frac / k_fixed, coverage >= 0 by mass coverage (sel's row length is the cap)."""
    B, max_pages = block_table.shape
    k_max = sel.shape[-1]
    rc = lib().kv_topk_sparse_decode_attn(
        ctypes.byref(L), _p(q), ctypes.byref(pages), _p(block_table), _p(seq_lens), int(B), int(max_pages),
        _p(head_scores), _p(lse_partial), float(keep_frac), int(k_fixed), float(coverage), int(n_force_first),
        int(n_force_last), _p(sel), _p(sel_count), int(k_max), _p(page_S), int(num_splits), _p(out), _p(lse),
        _p(ws), 0 if ws is None else ws.numel() * ws.element_size(), _stream(stream))
    _check(rc, "kv_topk_sparse_decode_attn")


def step_workspace_size(L, B, k_max, num_splits=0):
    return int(lib().kv_sparse_decode_step_workspace_size(ctypes.byref(L), int(B), int(k_max), int(num_splits)))


def step_supported(L, B, max_pages, k_max, num_splits=0):
    return bool(lib().kv_sparse_decode_step_supported(ctypes.byref(L), int(B), int(max_pages), int(k_max),
                                                      int(num_splits)))


def step_fused(L, pages, B, max_pages, k_max, num_splits=0):
    """Whether kv_sparse_decode_step takes the fused selector + attention launch here."""
    return bool(lib().kv_sparse_decode_step_fused(ctypes.byref(L), ctypes.byref(pages), int(B), int(max_pages),
                                                  int(k_max), int(num_splits)))


def sparse_decode_step(L, q, summary, log_n, pages, block_table, seq_lens, head_scores, lse_partial, sel,
                       sel_count, out, lse, ws, keep_frac=0.0, k_fixed=0, coverage=-1.0, n_force_first=0,
                       n_force_last=0, page_S=None, num_splits=0, stream=None):
    """Score, selection and sparse attention of one layer in one call (the
    faster of the fused and the separate schedules; outputs as kv_page_score
    followed by kv_topk_sparse_decode_attn)."""
    B, max_pages = block_table.shape
    k_max = sel.shape[-1]
    rc = lib().kv_sparse_decode_step(
        ctypes.byref(L), _p(q), _p(summary), _p(log_n), ctypes.byref(pages), _p(block_table), _p(seq_lens),
        int(B), int(max_pages), float(keep_frac), int(k_fixed), float(coverage), int(n_force_first),
        int(n_force_last), _p(head_scores), _p(lse_partial), _p(sel), _p(sel_count), int(k_max), _p(page_S),
        int(num_splits), _p(out), _p(lse), _p(ws), 0 if ws is None else ws.numel() * ws.element_size(),
        _stream(stream))
    _check(rc, "kv_sparse_decode_step")


def sparse_decode_step_noalloc(L, q, summary, log_n, pages, block_table, seq_lens, head_scores, lse_partial, sel,
                               sel_count, out, lse, keep_frac=0.0, k_fixed=0, coverage=-1.0, n_force_first=0,
                               n_force_last=0, page_S=None, num_splits=0, stream=None):
    """kv_sparse_decode_step with the attention's cross-block state in the
    library's own device array instead of a workspace (allocates nothing)."""
    B, max_pages = block_table.shape
    k_max = sel.shape[-1]
    rc = lib().kv_sparse_decode_step_noalloc(
        ctypes.byref(L), _p(q), _p(summary), _p(log_n), ctypes.byref(pages), _p(block_table), _p(seq_lens),
        int(B), int(max_pages), float(keep_frac), int(k_fixed), float(coverage), int(n_force_first),
        int(n_force_last), _p(head_scores), _p(lse_partial), _p(sel), _p(sel_count), int(k_max), _p(page_S),
        int(num_splits), _p(out), _p(lse), _stream(stream))
    _check(rc, "kv_sparse_decode_step_noalloc")


def dequant_tier(L, pages, page_ids, out, stream=None):
    rc = lib().kv_dequant_tier(ctypes.byref(L), ctypes.byref(pages), _p(page_ids), int(page_ids.numel()),
                               _p(out), _stream(stream))
    _check(rc, "kv_dequant_tier")


def pack_tier(L, src16, n, tier, codes, scale_zero, src_pages=None, dst_slots=None, stream=None, outliers=None):
    rc = lib().kv_pack_tier(ctypes.byref(L), _p(src16), _p(src_pages), int(n), int(tier), _p(codes),
                            _p(scale_zero), _p(outliers), _p(dst_slots), _stream(stream))
    _check(rc, "kv_pack_tier")
