"""Device-side set-up of a synthetic decode layer and one decode step through the C ABI.

Allocation and upload only (torch for device memory and streams); every step of
the method runs in libkvsparse.  Used by the GPU tests and bench.py.
"""

from __future__ import annotations

import ctypes
import math

import numpy as np
import torch

from . import kvsparse as kv
from . import workloads as wl

TORCH16 = {"bf16": torch.bfloat16, "f16": torch.float16}


def to_device16(bits, dtype, device="cuda"):
    """uint16 numpy bits -> torch 16-bit tensor on the device."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(TORCH16[dtype]).to(device)


def layout_of(w: wl.Workload, softmax_scale=0.0):
    return kv.layout(w.Hq, w.Hkv, w.d, w.P, w.rank, w.dtype, softmax_scale)


# ------------------------------------------------------------------ pinned, mapped host memory

class MappedHostBuffer:
    """hipHostMalloc(..., hipHostMallocMapped) buffer with its device address."""

    def __init__(self, nbytes):
        self._hip = ctypes.CDLL("libamdhip64.so")
        self.host = ctypes.c_void_p()
        rc = self._hip.hipHostMalloc(ctypes.byref(self.host), ctypes.c_size_t(nbytes), ctypes.c_uint(0x2))
        if rc != 0:
            raise RuntimeError(f"hipHostMalloc({nbytes}) failed: {rc}")
        self.dev = ctypes.c_void_p()
        rc = self._hip.hipHostGetDevicePointer(ctypes.byref(self.dev), self.host, ctypes.c_uint(0))
        if rc != 0:
            raise RuntimeError(f"hipHostGetDevicePointer failed: {rc}")
        self.nbytes = nbytes

    def numpy(self, dtype, shape):
        buf = (ctypes.c_char * self.nbytes).from_address(self.host.value)
        return np.frombuffer(buf, dtype=dtype).reshape(shape)

    def free(self):
        if self.host:
            self._hip.hipHostFree(self.host)
            self.host = ctypes.c_void_p()


# ------------------------------------------------------------------ one layer

class DeviceLayer:
    """K/V pools, block table, summaries (and tier pools / host V) of one layer."""

    def __init__(self, w: wl.Workload, layer=0, summaries="build", device="cuda", host_v=None,
                 hot_mode="warm", seq_lens=None, threads=None, host_k=None, tier_slots="compact",
                 b1_outliers=False):
        self.w, self.layer, self.device = w, layer, device
        self.L = layout_of(w)
        host_v = w.v_host if host_v is None else host_v
        host_k = w.k_host if host_k is None else host_k
        if host_k and (not host_v or w.tier_fracs is not None):
            raise ValueError("a host-resident K pool needs a host-resident V pool and native pages only")
        shape = (w.n_phys, w.Hkv, w.P, w.d)
        self.bt_np = wl.block_table(w, layer)
        self.bt = torch.from_numpy(self.bt_np).to(device)
        self.seq_lens_np = wl.seq_lens(w) if seq_lens is None else np.asarray(seq_lens, dtype=np.int32)
        self.seq_lens = torch.from_numpy(self.seq_lens_np).to(device)
        self.host_k = None
        if host_k:
            self.host_k = MappedHostBuffer(int(np.prod(shape)) * 2)
            kbits = self.host_k.numpy(np.uint16, shape)
        else:
            kbits = np.empty(shape, dtype=np.uint16)
        self.host_v = None
        if host_v:
            self.host_v = MappedHostBuffer(int(np.prod(shape)) * 2)
            vbits = self.host_v.numpy(np.uint16, shape)
        else:
            vbits = np.empty(shape, dtype=np.uint16)
        wl.fill_pools(w, layer, kbits, vbits, self.bt_np, threads=threads)
        # the K pool as the kernels take it: a device tensor, or the device
        # address of the mapped host pool
        self.k16 = None if host_k else to_device16(kbits, w.dtype, device)
        self.k_src = self.host_k.dev.value if host_k else self.k16
        del kbits
        self.v16 = None if host_v else to_device16(vbits, w.dtype, device)
        del vbits
        # summaries in logical page order per (sequence, KV head): per-page
        # directions ("build", "synthetic") or a shared row basis with per-page
        # means and variances ("basis_build", "basis_synthetic")
        self.summary = self.basis = self.mu = self.lam = None
        self.coords = self.lr_basis = self.lr_mean = None
        self.log_n = torch.empty((w.B, w.Np), dtype=torch.float32, device=device)
        if summaries in ("build", "synthetic"):
            self.summary = torch.empty((w.B, w.Hkv, w.Np, (1 + w.rank) * w.d), dtype=torch.bfloat16,
                                       device=device)
        elif summaries in ("basis_build", "basis_synthetic"):
            self.basis = torch.empty((w.B, w.Hkv, w.rank, w.d), dtype=torch.float32, device=device)
            self.mu = torch.empty((w.B, w.Hkv, w.Np, w.d), dtype=torch.bfloat16, device=device)
            self.lam = torch.empty((w.B, w.Hkv, w.Np, w.rank), dtype=torch.float32, device=device)
        if summaries == "build":
            self.build_summaries()
        elif summaries == "synthetic":
            rec, n_valid = wl.synthetic_summary(w, layer)
            self.summary.copy_(to_device16(rec.reshape(w.B, w.Hkv, w.Np, -1), "bf16", device))
            self.log_n.copy_(torch.from_numpy(np.log(n_valid.astype(np.float64)).astype(np.float32)))
        elif summaries in ("lowrank_build", "lowrank_synthetic"):
            self._alloc_lowrank()
            if summaries == "lowrank_build":
                self.build_lowrank()
            else:
                U, m, cbits = wl.synthetic_lowrank(w, layer, seq_lens_=self.seq_lens_np)
                self.lr_basis.copy_(torch.from_numpy(U))
                self.lr_mean.copy_(torch.from_numpy(m))
                self.coords.copy_(to_device16(cbits, "bf16", device))
        if summaries == "basis_build":
            self.build_basis()
            self.build_basis_summaries()
        elif summaries == "basis_synthetic":
            U, mu_bits, lam, n_valid = wl.synthetic_basis_summary(w, layer)
            self.basis.copy_(torch.from_numpy(U))
            self.mu.copy_(to_device16(mu_bits, "bf16", device))
            self.lam.copy_(torch.from_numpy(lam))
            self.log_n.copy_(torch.from_numpy(np.log(n_valid.astype(np.float64)).astype(np.float32)))
        self.tiers = None
        self.page_entry = None
        self.kout = self.vout = None
        if w.tier_fracs is not None:
            self._pack_tiers(tier_slots, b1_outliers)
        self.v_hot = self.k_hot = None
        self.v_hot_slot = None
        if host_v:
            self._init_hot_buffer(hot_mode)
        self.pages = self._make_pages()

    def valid_tokens(self):
        """(B, Np) valid tokens of every logical page under the current seq_lens."""
        w = self.w
        starts = np.arange(w.Np, dtype=np.int64) * w.P
        return np.clip(self.seq_lens_np[:, None].astype(np.int64) - starts[None, :], 0, w.P).astype(np.int32)

    # summary of every logical page, over its valid tokens (0 -> empty record)
    def build_summaries(self, stream=None):
        entries, nv = self._all_entries()
        kv.summary_build(self.L, self.k_src, self.bt, entries, nv, self.summary, self.log_n, stream)

    def with_basis_summaries(self, stream=None):
        """The same layer (pools, block table, tiers, host V shared) scored from
        shared-basis summaries built from its keys; release() the original only."""
        import copy
        w = self.w
        v = copy.copy(self)
        v.summary = None
        v.basis = torch.empty((w.B, w.Hkv, w.rank, w.d), dtype=torch.float32, device=self.device)
        v.mu = torch.empty((w.B, w.Hkv, w.Np, w.d), dtype=torch.bfloat16, device=self.device)
        v.lam = torch.empty((w.B, w.Hkv, w.Np, w.rank), dtype=torch.float32, device=self.device)
        v.log_n = torch.empty_like(self.log_n)
        v.host_v = v.host_k = None
        v.build_basis(stream)
        v.build_basis_summaries(stream)
        return v

    # r8 low-rank state: row basis (rank 8) and mean, per-key coordinates
    def _alloc_lowrank(self, rank=8):
        w = self.w
        self.L_lr = layout_of(w.replace(rank=rank))
        self.lr_basis = torch.empty((w.B, w.Hkv, rank, w.d), dtype=torch.float32, device=self.device)
        self.lr_mean = torch.empty((w.B, w.Hkv, w.d), dtype=torch.float32, device=self.device)
        self.coords = torch.zeros((w.B, w.Hkv, w.Np, w.P, rank), dtype=torch.bfloat16, device=self.device)

    def build_lowrank(self, stream=None):
        w = self.w
        nb = kv.basis_build_workspace_size(self.L_lr, w.B, w.Np)
        ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device=self.device)
        kv.basis_build(self.L_lr, self.k_src, self.bt, self.seq_lens, self.lr_basis, ws, stream, mean=self.lr_mean)
        entries, nv = self._all_entries()
        kv.lowrank_coords(self.L_lr, self.k_src, self.bt, entries, nv, self.lr_basis, self.lr_mean, self.coords,
                          stream)
        if stream is None:
            torch.cuda.current_stream().synchronize()
        del ws

    def with_lowrank_summaries(self, stream=None):
        """The same layer scored with the r8 low-rank score built from its keys;
        release() the original only."""
        import copy
        v = copy.copy(self)
        v.summary = v.basis = v.mu = v.lam = None
        v.host_v = v.host_k = None
        v._alloc_lowrank()
        v.build_lowrank(stream)
        return v

    def _all_entries(self):
        w = self.w
        bb, pp = np.meshgrid(np.arange(w.B), np.arange(w.Np), indexing="ij")
        entries = torch.from_numpy(np.stack([bb.ravel(), pp.ravel()], 1).astype(np.int32)).to(self.device)
        nv = torch.from_numpy(self.valid_tokens().ravel()).to(self.device)
        return entries, nv

    # the row basis over every valid key (prefill)
    def build_basis(self, stream=None):
        w = self.w
        nb = kv.basis_build_workspace_size(self.L, w.B, w.Np)
        ws = torch.empty(max(1, nb // 4), dtype=torch.float32, device=self.device)
        kv.basis_build(self.L, self.k_src, self.bt, self.seq_lens, self.basis, ws, stream)
        if stream is None:
            torch.cuda.current_stream().synchronize()
        del ws

    # shared-basis statistics of every logical page (0 valid tokens -> zeros)
    def build_basis_summaries(self, stream=None):
        entries, nv = self._all_entries()
        kv.summary_build_basis(self.L, self.k_src, self.bt, entries, nv, self.basis, self.mu, self.lam,
                               self.log_n, stream)

    def _pack_tiers(self, tier_slots="compact", b1_outliers=False):
        """Packs every page into its tier.  tier_slots "compact": a tier's pool
        holds only its pages; "phys": every tier pool has a slot per physical
        page and a page sits at slot = its physical id (what tier demotion
        writes to).  b1_outliers: the 1-bit tier keeps outlier side tables."""
        w = self.w
        tiers_logical = wl.page_tiers(w, self.layer)              # (B, Np)
        tier_phys = np.zeros(w.n_phys, dtype=np.int64)
        tier_phys[self.bt_np.ravel()] = tiers_logical.ravel()
        self.tier_phys = tier_phys
        entry = np.zeros(w.n_phys, dtype=np.uint32)
        self.kq, self.vq, self.ksz, self.vsz = [], [], [], []
        full = tier_slots == "phys"
        for t in range(1, kv.NUM_PACKED_TIERS + 1):
            phys = np.nonzero(tier_phys == t)[0].astype(np.int32)
            n = w.n_phys if full else max(1, phys.size)
            bits = kv.TIER_BITS[t]
            kc = torch.zeros((n, w.Hkv, w.P, w.d * bits // 8), dtype=torch.uint8, device=self.device)
            vc = torch.zeros_like(kc)
            ks = torch.zeros((n, w.Hkv, w.P, w.d // 32, 2), dtype=torch.float16, device=self.device)
            vs = torch.zeros_like(ks)
            ko = vo = None
            if b1_outliers and t == kv.KV_TIER_B1:
                ko = torch.zeros((n, w.Hkv, w.P, w.d // 32), dtype=torch.int32, device=self.device)
                vo = torch.zeros_like(ko)
                self.kout, self.vout = ko, vo
            if phys.size:
                src = torch.from_numpy(phys).to(self.device)
                slots = phys if full else np.arange(phys.size, dtype=np.int32)
                dst = torch.from_numpy(slots).to(self.device) if full else None
                kv.pack_tier(self.L, self.k16, phys.size, t, kc, ks, src_pages=src, dst_slots=dst, outliers=ko)
                kv.pack_tier(self.L, self.v16, phys.size, t, vc, vs, src_pages=src, dst_slots=dst, outliers=vo)
                entry[phys] = (np.uint32(t) << np.uint32(29)) | slots.astype(np.uint32)
            self.kq.append(kc); self.vq.append(vc); self.ksz.append(ks); self.vsz.append(vs)
        native = np.nonzero(tier_phys == 0)[0]
        entry[native] = native.astype(np.uint32)                  # native slot = physical page
        self.page_entry = torch.from_numpy(entry.view(np.int32)).to(self.device)
        self.tiers = tier_phys

    def _init_hot_buffer(self, hot_mode):
        """HBM hot buffer of hot_buffer_frac of the (physical page, KV head)
        units, seeded random contents."""
        w = self.w
        n_slots = max(1, int(round(w.hot_buffer_frac * w.n_phys * w.Hkv)))
        self.n_hot = n_slots
        self.v_hot = torch.empty((n_slots, w.P, w.d), dtype=TORCH16[w.dtype], device=self.device)
        if self.host_k is not None:
            self.k_hot = torch.empty_like(self.v_hot)
        self.set_hot_units(np.zeros(0, np.int64), fill_random=True)

    def set_hot_units(self, must_include, fill_random=True):
        """Hot buffer = must_include units u = phys * Hkv + g (then a seeded
        random fill); copies their V (and K with a host K pool)."""
        w = self.w
        slot, chosen = wl.hot_buffer_slots(w, self.n_hot if fill_random else min(self.n_hot, len(must_include)),
                                           self.layer, must_include)
        self.v_hot_slot = torch.from_numpy(slot).to(self.device)
        vh = self.host_v.numpy(np.uint16, (w.n_phys * w.Hkv, w.P, w.d))
        stage = torch.from_numpy(np.ascontiguousarray(vh[chosen]).view(np.int16)).view(TORCH16[w.dtype])
        self.v_hot[: len(chosen)].copy_(stage.to(self.device))
        if self.host_k is not None:
            kh = self.host_k.numpy(np.uint16, (w.n_phys * w.Hkv, w.P, w.d))
            stage = torch.from_numpy(np.ascontiguousarray(kh[chosen]).view(np.int16)).view(TORCH16[w.dtype])
            self.k_hot[: len(chosen)].copy_(stage.to(self.device))
        self.hot_units = chosen
        self.pages = self._make_pages()

    def _make_pages(self):
        v16 = self.v16
        v16_ptr = self.host_v.dev.value if self.host_v is not None else None
        if self.page_entry is not None:
            return kv.make_pages(self.k16, v16, self.kq, self.vq, self.ksz, self.vsz, self.page_entry,
                                 self.v_hot, self.v_hot_slot, v16_ptr=v16_ptr, kout=self.kout, vout=self.vout)
        return kv.make_pages(self.k16, v16, page_entry=None, v_hot=self.v_hot, v_hot_slot=self.v_hot_slot,
                             v16_ptr=v16_ptr, k_hot=self.k_hot,
                             k16_ptr=self.host_k.dev.value if self.host_k is not None else None)

    def release(self):
        if self.host_v is not None or self.host_k is not None:
            torch.cuda.synchronize()
        for name in ("host_v", "host_k"):
            buf = getattr(self, name)
            if buf is not None:
                buf.free()
                setattr(self, name, None)


# ------------------------------------------------------------------ step buffers

class StepBuffers:
    def __init__(self, w: wl.Workload, device="cuda", num_splits=0, with_S=False):
        L = layout_of(w)
        self.k_max = w.k_of(w.Np)
        self.num_splits = num_splits
        self.head_scores = torch.empty((w.B, w.Hkv, w.G, w.Np), dtype=torch.float32, device=device)
        nb = kv.page_score_partial_size(L, w.B, w.Np)
        self.lse_partial = torch.empty(nb // 4, dtype=torch.float32, device=device)
        self.sel = torch.empty((w.B, w.Hkv, max(1, self.k_max)), dtype=torch.int32, device=device)
        self.sel_count = torch.empty((w.B, w.Hkv), dtype=torch.int32, device=device)
        self.page_S = torch.empty((w.B, w.Hkv, w.Np), dtype=torch.float32, device=device) if with_S else None
        self.out = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device=device)
        self.lse = torch.empty((w.B, w.Hq), dtype=torch.float32, device=device)
        nws = kv.attn_workspace_size(L, w.B, self.sel.shape[-1], num_splits)
        # zeroed once: its per-row counters must start at zero (each call leaves them at zero)
        self.ws = torch.zeros(max(1, nws // 4), dtype=torch.float32, device=device)


def queries_device(w: wl.Workload, layer=0, qidx=0, device="cuda"):
    return to_device16(wl.query_tensor(w, layer, qidx), w.dtype, device)


def drift_queries_device(w: wl.Workload, n_steps: int, c: float, layer=0, device="cuda"):
    """n_steps [B, Hq, d] 16-bit device tensors of wl.drift_queries (every row)."""
    rows = np.stack([np.stack([wl.drift_queries(w, layer, b, g, n_steps, c) for g in range(w.Hkv)], 1)
                     for b in range(w.B)], 1)           # (n_steps, B, Hkv, G, d)
    rows = rows.reshape(n_steps, w.B, w.Hq, w.d)
    return [to_device16(wl.to_bits(rows[t], w.dtype), w.dtype, device) for t in range(n_steps)]


def score(layer: DeviceLayer, q, bufs: StepBuffers, stream=None):
    if layer.coords is not None:
        kv.page_score_lowrank(layer.L_lr, q, layer.coords, layer.lr_mean, layer.lr_basis, layer.seq_lens,
                              bufs.head_scores, bufs.lse_partial, stream)
    elif layer.basis is not None:
        kv.page_score_basis(layer.L, q, layer.mu, layer.lam, layer.basis, layer.log_n, layer.seq_lens,
                            bufs.head_scores, bufs.lse_partial, stream)
    else:
        kv.page_score(layer.L, q, layer.summary, layer.log_n, layer.seq_lens, bufs.head_scores,
                      bufs.lse_partial, stream)


def topk(layer: DeviceLayer, bufs: StepBuffers, n_force_first=0, n_force_last=0, stream=None):
    w = layer.w
    kv.page_topk(layer.L, bufs.head_scores, bufs.lse_partial, layer.seq_lens, w.Np, w.keep, w.k_fixed,
                 bufs.sel, bufs.sel_count, n_force_first, n_force_last, bufs.page_S, None, stream)


def attend(layer: DeviceLayer, q, bufs: StepBuffers, sel=None, sel_count=None, stream=None):
    kv.sparse_decode_attn(layer.L, q, layer.pages, layer.bt, layer.seq_lens,
                          bufs.sel if sel is None else sel, bufs.sel_count if sel_count is None else sel_count,
                          bufs.out, bufs.lse, bufs.ws, bufs.num_splits, stream)


def fused_supported(layer: DeviceLayer, bufs: StepBuffers):
    w = layer.w
    s = bufs.num_splits or kv.attn_num_splits(layer.L, w.B, bufs.sel.shape[-1], layer.page_entry is not None)
    return kv.topk_attn_supported(layer.L, w.Np, bufs.sel.shape[-1], s)


def fused_preferred(layer: DeviceLayer, bufs: StepBuffers):
    """Where the fused top-k + attention call is the faster step: native pages,
    up to four query heads per KV head (eight-wave blocks) and rows under 4096
    pages.  Packed tiers want two blocks per CU, and long rows or wider groups
    select too slowly inside one block; there the separate launches win."""
    w = layer.w
    return (layer.page_entry is None and w.G <= 4 and w.Np < 4096 and fused_supported(layer, bufs))


def topk_attend(layer: DeviceLayer, q, bufs: StepBuffers, n_force_first=0, n_force_last=0, coverage=-1.0,
                stream=None):
    """top-k and sparse attention in one launch (the same results as topk + attend)."""
    w = layer.w
    kv.topk_sparse_decode_attn(layer.L, q, layer.pages, layer.bt, layer.seq_lens, bufs.head_scores,
                               bufs.lse_partial, bufs.sel, bufs.sel_count, bufs.out, bufs.lse, bufs.ws,
                               keep_frac=w.keep, k_fixed=w.k_fixed, coverage=coverage,
                               n_force_first=n_force_first, n_force_last=n_force_last, page_S=bufs.page_S,
                               num_splits=bufs.num_splits, stream=stream)


def step_supported(layer: DeviceLayer, bufs: StepBuffers):
    """Whether kv_sparse_decode_step takes this layer (quad summaries)."""
    w = layer.w
    return (layer.summary is not None and layer.coords is None and layer.basis is None and
            kv.step_supported(layer.L, w.B, w.Np, bufs.sel.shape[-1], bufs.num_splits))


def whole_step(layer: DeviceLayer, q, bufs: StepBuffers, n_force_first=0, n_force_last=0, coverage=-1.0,
               stream=None):
    """score, top-k and sparse attention in one library call (kv_sparse_decode_step)."""
    w = layer.w
    kv.sparse_decode_step(layer.L, q, layer.summary, layer.log_n, layer.pages, layer.bt, layer.seq_lens,
                          bufs.head_scores, bufs.lse_partial, bufs.sel, bufs.sel_count, bufs.out, bufs.lse,
                          bufs.ws, keep_frac=w.keep, k_fixed=w.k_fixed, coverage=coverage,
                          n_force_first=n_force_first, n_force_last=n_force_last, page_S=bufs.page_S,
                          num_splits=bufs.num_splits, stream=stream)


def decode_step(layer: DeviceLayer, q, bufs: StepBuffers, stream=None, fused=False):
    """score -> top-k -> sparse attention for one layer of the whole batch
    (fused: top-k and attention in one launch; "step": kv_sparse_decode_step)."""
    if fused == "step":
        whole_step(layer, q, bufs, stream=stream)
        return
    score(layer, q, bufs, stream)
    if fused:
        topk_attend(layer, q, bufs, stream=stream)
    else:
        topk(layer, bufs, stream=stream)
        attend(layer, q, bufs, stream=stream)


# ------------------------------------------------------------------ overlapped row groups

class _View:
    pass


class SplitStep:
    """One decode step with the batch cut into row groups, each group's
    score -> top-k -> attention chain on its own HIP stream.

    Rows are independent, so a group's selection and attention can run while
    another group is still being scored; the C ABI is called per group with
    pointers offset to that group's sequences (no library change).  All
    streams keep the default priority."""

    def __init__(self, layer: DeviceLayer, bufs: StepBuffers, n_groups=2, num_splits=0, fused=False):
        w = layer.w
        self.layer, self.bufs = layer, bufs
        self.fused = fused
        n_groups = max(1, min(n_groups, w.B))
        edges = [round(i * w.B / n_groups) for i in range(n_groups + 1)]
        self.streams = [torch.cuda.Stream() for _ in range(n_groups)]
        lp = bufs.lse_partial.view(w.B, -1)
        self.groups = []
        for b0, b1 in zip(edges[:-1], edges[1:]):
            v = _View()
            v.b0, v.b1 = b0, b1
            v.summary = None if layer.summary is None else layer.summary[b0:b1]
            v.basis = None if layer.basis is None else layer.basis[b0:b1]
            v.mu = None if layer.mu is None else layer.mu[b0:b1]
            v.lam = None if layer.lam is None else layer.lam[b0:b1]
            v.log_n = layer.log_n[b0:b1]
            v.seq_lens = layer.seq_lens[b0:b1]
            v.bt = layer.bt[b0:b1]
            v.head_scores = bufs.head_scores[b0:b1]
            v.lse_partial = lp[b0:b1]
            v.sel = bufs.sel[b0:b1]
            v.sel_count = bufs.sel_count[b0:b1]
            v.page_S = None if bufs.page_S is None else bufs.page_S[b0:b1]
            v.out = bufs.out[b0:b1]
            v.lse = bufs.lse[b0:b1]
            nws = kv.attn_workspace_size(layer.L, b1 - b0, bufs.sel.shape[-1], num_splits)
            v.ws = torch.zeros(max(1, nws // 4), dtype=torch.float32, device=layer.device)
            self.groups.append(v)
        self.num_splits = num_splits

    def __call__(self, q):
        layer, w = self.layer, self.layer.w
        main = torch.cuda.current_stream()
        for s in self.streams:
            s.wait_stream(main)
        for v, s in zip(self.groups, self.streams):
            with torch.cuda.stream(s):
                qg = q[v.b0:v.b1]
                if v.basis is not None:
                    kv.page_score_basis(layer.L, qg, v.mu, v.lam, v.basis, v.log_n, v.seq_lens, v.head_scores,
                                        v.lse_partial, s)
                else:
                    kv.page_score(layer.L, qg, v.summary, v.log_n, v.seq_lens, v.head_scores, v.lse_partial, s)
                if self.fused:
                    kv.topk_sparse_decode_attn(layer.L, qg, layer.pages, v.bt, v.seq_lens, v.head_scores,
                                               v.lse_partial, v.sel, v.sel_count, v.out, v.lse, v.ws,
                                               keep_frac=w.keep, k_fixed=w.k_fixed, page_S=v.page_S,
                                               num_splits=self.num_splits, stream=s)
                    continue
                kv.page_topk(layer.L, v.head_scores, v.lse_partial, v.seq_lens, w.Np, w.keep, w.k_fixed,
                             v.sel, v.sel_count, 0, 0, v.page_S, None, s)
                kv.sparse_decode_attn(layer.L, qg, layer.pages, v.bt, v.seq_lens, v.sel, v.sel_count,
                                      v.out, v.lse, v.ws, self.num_splits, s)
        for s in self.streams:
            main.wait_stream(s)


# ------------------------------------------------------------------ host-resident pool with admission

class MemStep:
    """Decode steps over a layer whose V (and, with a host K pool, K) lives in
    device-mapped host memory behind an HBM hot buffer of (page, KV head)
    units.

    Per step, on the caller's stream: score, top-k, then (with admit=True)
    kv_hot_admit, which stamps the units the selection calls that are hot and
    copies the others into the least recently used slots, then attention,
    which so reads every admitted unit from HBM.  With admit=False the hot
    buffer stays as the layer set it up and attention reads the units that
    are not hot over the host link."""

    def __init__(self, layer: DeviceLayer, admit=True):
        w = layer.w
        if layer.v_hot is None:
            raise ValueError("MemStep needs a layer with a host-resident pool and a hot buffer")
        self.layer, self.admit = layer, admit
        self.bufs = [StepBuffers(w, layer.device), StepBuffers(w, layer.device)]
        n_slots = layer.v_hot.shape[0]
        sp = np.full(n_slots, -1, dtype=np.int32)
        sp[: len(layer.hot_units)] = np.asarray(layer.hot_units, dtype=np.int32)
        self.slot_page = torch.from_numpy(sp).to(layer.device)
        self.slot_stamp = torch.zeros(n_slots, dtype=torch.int32, device=layer.device)
        self.ws = torch.zeros(kv.hot_admit_workspace_size(n_slots, layer.v_hot_slot.shape[0]) // 4,
                              dtype=torch.int32, device=layer.device)
        self.admit_start = torch.cuda.Event(enable_timing=True)
        self.admitted = torch.cuda.Event(enable_timing=True)
        self.t = 0

    def admit_step(self, bufs, stream=None):
        layer = self.layer
        kv.hot_admit(layer.L, layer.host_v.dev.value, layer.v_hot, layer.v_hot_slot, self.slot_page,
                     self.slot_stamp, layer.bt, layer.seq_lens, bufs.sel, bufs.sel_count, self.t, self.ws, stream,
                     k16_ptr=layer.host_k.dev.value if layer.host_k is not None else None, k_hot=layer.k_hot)

    def __call__(self, q):
        layer = self.layer
        bufs = self.bufs[self.t & 1]
        score(layer, q, bufs)
        topk(layer, bufs)
        self.t += 1
        if self.admit:
            self.admit_step(bufs)
        attend(layer, q, bufs)
        return bufs

