"""Seeded synthetic decode workloads (inputs only; none of the method's arithmetic).

Shapes follow the long-context decode settings the AMASS page describes
(amass-kv 0.1.1 project page, section "AMASS": a small working set of pages per
step at long context) and the packed tiers of the ARGUS page (argus_cache
0.1.7.1 project page, section "Visual Architecture").  No dataset or model
weights are used: every tensor is drawn from a fixed distribution.

Every (layer, sequence, KV head, tensor) draws from its own numpy
``Generator(PCG64(SeedSequence([seed, workload id, layer, b, g, tensor, extra])))``
so any single row can be regenerated without materialising the rest.  Values
are rounded to the workload's 16-bit dtype (round to nearest even) and handed
out as float32 arrays holding those exact values, or as uint16 bit patterns.

This module serves both the GPU path's tests and bench and the CPU oracle's
tests.  It only draws random numbers and arranges them.
"""

from __future__ import annotations

import concurrent.futures as cf
import dataclasses
import math
import os

import numpy as np

SEED = 2026

T_Q, T_K, T_V, T_HOT, T_TABLE, T_TIER, T_SEL, T_SUMMARY, T_CENTERS, T_HOTBUF, T_BASIS, T_LOWRANK, T_DRIFT = range(13)

TIER_NAMES = ("native", "int8", "int4", "int2", "1bit", "fp8")


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    wid: int
    B: int
    Hq: int
    Hkv: int
    d: int
    P: int
    ctx: int
    rank: int
    keep: float
    k_fixed: int
    dtype: str                    # "f16" | "bf16"
    keys: str                     # "planted" | "hot" | "gmm"
    n_hot: int = 0                # planted pages per sequence ("planted")
    hot_frac: float = 0.0         # planted page fraction per sequence ("hot")
    sink: bool = False            # page 0 planted as well
    plant_scale: float = 2.5
    gmm_centers: int = 0
    gmm_std: float = 0.0
    tier_fracs: tuple | None = None   # fractions per tier, most to least important
    tier_order: tuple = (0, 1, 2, 3, 4)   # tier id of each fraction (5 = fp8)
    v_host: bool = False          # V pool in pinned host memory, read through a mapping
    k_host: bool = False          # K pool there too (mem-kv; needs v_host)
    hot_buffer_frac: float = 0.0  # HBM hot buffer for V, fraction of physical pages

    @property
    def G(self):
        return self.Hq // self.Hkv

    @property
    def Np(self):
        return -(-self.ctx // self.P)

    @property
    def rows(self):
        return self.B * self.Hkv

    @property
    def n_phys(self):
        return self.B * self.Np

    @property
    def tau(self):
        return 1.0 / math.sqrt(self.d)

    def k_of(self, npages):
        if npages <= 0:
            return 0
        if self.k_fixed > 0:
            return min(npages, self.k_fixed)
        return min(npages, max(1, math.ceil(float(np.float32(self.keep)) * npages)))

    def replace(self, **kw):
        return dataclasses.replace(self, **kw)


WORKLOADS = {
    w.name: w for w in [
        Workload("tiny", 0, B=1, Hq=8, Hkv=2, d=64, P=16, ctx=1024, rank=2, keep=0.125, k_fixed=8,
                 dtype="f16", keys="planted", n_hot=4, plant_scale=3.0),
        Workload("llama8b_32k", 1, B=8, Hq=32, Hkv=8, d=128, P=16, ctx=32768, rank=4, keep=0.08,
                 k_fixed=0, dtype="bf16", keys="hot", hot_frac=0.02, sink=True, plant_scale=2.5),
        Workload("tiers_64k", 2, B=4, Hq=32, Hkv=8, d=128, P=16, ctx=65536, rank=4, keep=0.10,
                 k_fixed=0, dtype="bf16", keys="hot", hot_frac=0.02, sink=True, plant_scale=2.5,
                 tier_fracs=(0.05, 0.15, 0.30, 0.40, 0.10)),
        Workload("qwen3b_128k", 3, B=16, Hq=16, Hkv=2, d=128, P=16, ctx=131072, rank=4, keep=0.05,
                 k_fixed=0, dtype="bf16", keys="gmm", gmm_centers=64, gmm_std=0.5),
        # the tiered shape with the cascade's FP8 step added (native, fp8, int8,
        # int4, int2, 1-bit)
        Workload("tiers_fp8_64k", 5, B=4, Hq=32, Hkv=8, d=128, P=16, ctx=65536, rank=4, keep=0.10,
                 k_fixed=0, dtype="bf16", keys="hot", hot_frac=0.02, sink=True, plant_scale=2.5,
                 tier_fracs=(0.05, 0.10, 0.15, 0.25, 0.35, 0.10), tier_order=(0, 5, 1, 2, 3, 4)),
        Workload("heavy70b_128k", 4, B=32, Hq=64, Hkv=8, d=128, P=32, ctx=131072, rank=4, keep=0.10,
                 k_fixed=0, dtype="bf16", keys="hot", hot_frac=0.01, plant_scale=2.5,
                 v_host=True, hot_buffer_frac=0.10),
    ]
}


def rng_for(w: Workload, layer: int, b: int, g: int, tensor: int, extra: int = 0):
    ss = np.random.SeedSequence([SEED, w.wid, layer, b, g, tensor, extra])
    return np.random.Generator(np.random.PCG64(ss))


# ---------------------------------------------------------------- 16-bit values

def bf16_bits(x32):
    """Round float32 to bfloat16 (nearest even) and return the uint16 bit patterns."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32)
    r = ((u >> 16) & 1) + np.uint32(0x7FFF)
    return ((u + r) >> 16).astype(np.uint16)


def bits_to_f32(bits, dtype):
    bits = np.asarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (bits.astype(np.uint32) << 16).view(np.float32)
    return bits.view(np.float16).astype(np.float32)


def to_bits(x32, dtype):
    if dtype == "bf16":
        return bf16_bits(x32)
    return np.asarray(x32, dtype=np.float32).astype(np.float16).view(np.uint16)


def round16(x32, dtype):
    """float32 values rounded to the 16-bit dtype, returned as float32."""
    return bits_to_f32(to_bits(x32, dtype), dtype)


# ---------------------------------------------------------------- per-row tensors

def queries(w: Workload, layer: int, b: int, g: int, qidx: int = 0):
    """(G, d) float32, the group of query heads attached to KV head g."""
    x = rng_for(w, layer, b, g, T_Q, qidx).standard_normal((w.G, w.d), dtype=np.float32)
    return round16(x, w.dtype)


def drift_queries(w: Workload, layer: int, b: int, g: int, n_steps: int, c: float):
    """(n_steps, G, d) float32 decode-step queries with step-to-step locality:
    q_0 is query draw 0 and q_t = c q_{t-1} + sqrt(1 - c^2) xi_t with seeded
    xi_t ~ N(0, 1), so every q_t is N(0, 1) per element and consecutive
    queries have cosine about c; each rounded to the pool dtype."""
    rng = rng_for(w, layer, b, g, T_DRIFT)
    x = queries(w, layer, b, g, 0).astype(np.float64)
    s = np.sqrt(max(0.0, 1.0 - c * c))
    out = np.empty((n_steps, w.G, w.d), dtype=np.float32)
    for t in range(n_steps):
        if t > 0:
            x = c * x + s * rng.standard_normal((w.G, w.d))
        out[t] = round16(x.astype(np.float32), w.dtype)
    return out


def hot_pages(w: Workload, layer: int, b: int):
    """Sorted logical pages that carry planted high-mass keys in sequence b."""
    rng = rng_for(w, layer, b, 0, T_HOT)
    if w.keys == "planted":
        n = w.n_hot
    elif w.keys == "hot":
        n = int(round(w.hot_frac * w.Np))
    else:
        n = 0
    pages = set(rng.choice(w.Np, size=n, replace=False).tolist()) if n else set()
    if w.sink:
        pages.add(0)
    return np.array(sorted(pages), dtype=np.int64)


def plant_direction(w: Workload, layer: int, b: int, g: int):
    """Unit vector along the sum of the group's queries (query draw 0)."""
    u = queries(w, layer, b, g, 0).astype(np.float64).sum(axis=0)
    return u / np.linalg.norm(u)


def row_keys(w: Workload, layer: int, b: int, g: int):
    """(Np*P, d) float32 keys of one (sequence, KV head), logical token order.

    Rows cover whole pages; tokens at or beyond ctx fill the last page's unused
    slots and are never valid."""
    rng = rng_for(w, layer, b, g, T_K)
    if w.keys == "gmm":
        centers = rng_for(w, layer, b, g, T_CENTERS).standard_normal((w.gmm_centers, w.d), dtype=np.float32)
        assign = rng.integers(0, w.gmm_centers, w.Np * w.P)
        x = centers[assign] + np.float32(w.gmm_std) * rng.standard_normal((w.Np * w.P, w.d), dtype=np.float32)
    else:
        x = rng.standard_normal((w.Np * w.P, w.d), dtype=np.float32)
        hp = hot_pages(w, layer, b)
        if hp.size:
            u = (w.plant_scale * plant_direction(w, layer, b, g)).astype(np.float32)
            xv = x.reshape(w.Np, w.P, w.d)
            xv[hp] += u
    return round16(x, w.dtype)


def row_values(w: Workload, layer: int, b: int, g: int):
    x = rng_for(w, layer, b, g, T_V).standard_normal((w.Np * w.P, w.d), dtype=np.float32)
    return round16(x, w.dtype)


# ---------------------------------------------------------------- paging metadata

def block_table(w: Workload, layer: int = 0):
    """(B, Np) int32: a seeded permutation of the physical pages (fragmented pool)."""
    perm = rng_for(w, layer, 0, 0, T_TABLE).permutation(w.n_phys).astype(np.int32)
    return perm.reshape(w.B, w.Np)


def seq_lens(w: Workload):
    return np.full(w.B, w.ctx, dtype=np.int32)


def page_tiers(w: Workload, layer: int = 0):
    """(B, Np) int8 tier per logical page, or None.

    A seeded uniform importance per page; within each sequence pages are cut by
    importance quantile, most important first, into the tier fractions.
    """
    if w.tier_fracs is None:
        return None
    out = np.zeros((w.B, w.Np), dtype=np.int8)
    bounds = np.floor(np.cumsum(w.tier_fracs) * w.Np + 1e-9).astype(np.int64)
    bounds[-1] = w.Np
    for b in range(w.B):
        imp = rng_for(w, layer, b, 0, T_TIER).random(w.Np)
        order = np.argsort(-imp, kind="stable")
        lo = 0
        for i, hi in enumerate(bounds):
            out[b, order[lo:hi]] = w.tier_order[i]
            lo = hi
    return out


def hot_buffer_slots(w: Workload, n_slots: int, layer: int = 0, must_include=()):
    """Units u = phys * Hkv + g (one physical page of one KV head) resident in
    the V hot buffer: must_include first, then a seeded random fill, at most
    n_slots.  Returns (slot_of_unit[n_phys * Hkv] int32, units)."""
    n_units = w.n_phys * w.Hkv
    rng = rng_for(w, layer, 0, 0, T_HOTBUF)
    chosen = list(dict.fromkeys(int(u) for u in must_include))[:n_slots]
    if len(chosen) < n_slots:
        rest = np.setdiff1d(rng.permutation(n_units), np.array(chosen, dtype=np.int64), assume_unique=False)
        rest = rng.permutation(rest)[: n_slots - len(chosen)]
        chosen += [int(u) for u in rest]
    slot = np.full(n_units, -1, dtype=np.int32)
    slot[np.array(chosen, dtype=np.int64)] = np.arange(len(chosen), dtype=np.int32)
    return slot, np.array(chosen, dtype=np.int64)


def synthetic_selection(w: Workload, k: int, layer: int = 0, ragged: bool = False):
    """(B, Hkv, k) int32 sorted distinct logical pages and counts (B, Hkv).

    With ragged=True every row keeps a seeded number of pages in [0, k]."""
    sel = np.full((w.B, w.Hkv, k), -1, dtype=np.int32)
    cnt = np.zeros((w.B, w.Hkv), dtype=np.int32)
    for b in range(w.B):
        for g in range(w.Hkv):
            rng = rng_for(w, layer, b, g, T_SEL)
            kk = int(rng.integers(0, k + 1)) if ragged else k
            kk = min(kk, w.Np)
            pick = np.sort(rng.choice(w.Np, size=kk, replace=False))
            sel[b, g, :kk] = pick
            cnt[b, g] = kk
    return sel, cnt


def synthetic_summary(w: Workload, layer: int = 0, lam=(12.0, 10.0, 9.0, 8.0, 7.0, 6.0, 5.0, 4.0)):
    """Random stored summaries shaped like real ones, for score/select tests.

    Returns (records uint16 [B, Hkv, Np, 1+rank, d] bf16 bits in logical page
    order, n_valid int32 [B, Np]).  mu ~ N(0, 1/P); direction j ~ N(0, lam_j/d);
    the planted pages carry a mean along their group's query direction."""
    rng = rng_for(w, layer, 0, 0, T_SUMMARY)
    rec = np.empty((w.B, w.Hkv, w.Np, 1 + w.rank, w.d), dtype=np.float32)
    rec[:, :, :, 0] = rng.standard_normal((w.B, w.Hkv, w.Np, w.d), dtype=np.float32) / np.float32(math.sqrt(w.P))
    for j in range(w.rank):
        sd = np.float32(math.sqrt(lam[j % len(lam)] / w.d))
        rec[:, :, :, 1 + j] = rng.standard_normal((w.B, w.Hkv, w.Np, w.d), dtype=np.float32) * sd
    for b in range(w.B):
        hp = hot_pages(w, layer, b)
        if hp.size:
            for g in range(w.Hkv):
                rec[b, g, hp, 0] += np.float32(w.plant_scale) * plant_direction(w, layer, b, g).astype(np.float32)
    n_valid = np.full((w.B, w.Np), w.P, dtype=np.int32)
    return bf16_bits(rec), n_valid


def synthetic_basis_summary(w: Workload, layer: int = 0, lam_scale=(3.0, 2.0, 1.5, 1.2, 1.0, 0.9, 0.8, 0.7)):
    """Random stored shared-basis summaries, for score/select tests.

    Returns (basis float32 [B, Hkv, rank, d] with orthonormal rows before
    rounding, mu uint16 bf16 bits [B, Hkv, Np, d] in logical page order,
    lam float32 [B, Hkv, Np, rank] >= 0, n_valid int32 [B, Np]).  mu is drawn as
    in synthetic_summary (planted pages carry a mean along their group's query
    direction); lam_j = lam_scale_j * (chi-square with P degrees of freedom) / P."""
    rng = rng_for(w, layer, 0, 0, T_BASIS)
    basis = np.empty((w.B, w.Hkv, w.rank, w.d), dtype=np.float32)
    for b in range(w.B):
        for g in range(w.Hkv):
            Q, _ = np.linalg.qr(rng.standard_normal((w.d, w.rank)))
            basis[b, g] = Q.T.astype(np.float32)
    mu = rng.standard_normal((w.B, w.Hkv, w.Np, w.d), dtype=np.float32) / np.float32(math.sqrt(w.P))
    for b in range(w.B):
        hp = hot_pages(w, layer, b)
        if hp.size:
            for g in range(w.Hkv):
                mu[b, g, hp] += np.float32(w.plant_scale) * plant_direction(w, layer, b, g).astype(np.float32)
    scale = np.array([lam_scale[j % len(lam_scale)] for j in range(w.rank)], dtype=np.float32)
    lam = (rng.chisquare(w.P, (w.B, w.Hkv, w.Np, w.rank)).astype(np.float32) / np.float32(w.P)) * scale
    n_valid = np.full((w.B, w.Np), w.P, dtype=np.int32)
    return basis, bf16_bits(mu), lam.astype(np.float32), n_valid


def synthetic_lowrank(w: Workload, layer: int = 0, rank: int = 8, seq_lens_=None):
    """Random stored low-rank (r8) state, for score/select tests.

    Returns (basis float32 [B, Hkv, rank, d] with orthonormal rows before
    rounding, mean float32 [B, Hkv, d], coords uint16 bf16 bits
    [B, Hkv, Np, P, rank]; tokens past a row's length hold 0).  Coordinates are
    N(0, 1) scaled by 1.5 / sqrt(j + 1) along direction j; planted pages get
    their first coordinate raised by 2, so they carry more mass."""
    rng = rng_for(w, layer, 0, 0, T_LOWRANK)
    lens = seq_lens(w) if seq_lens_ is None else np.asarray(seq_lens_)
    basis = np.empty((w.B, w.Hkv, rank, w.d), dtype=np.float32)
    for b in range(w.B):
        for g in range(w.Hkv):
            Q, _ = np.linalg.qr(rng.standard_normal((w.d, rank)))
            basis[b, g] = Q.T.astype(np.float32)
    mean = (0.3 * rng.standard_normal((w.B, w.Hkv, w.d))).astype(np.float32)
    scale = (1.5 / np.sqrt(np.arange(1, rank + 1))).astype(np.float32)
    c = rng.standard_normal((w.B, w.Hkv, w.Np, w.P, rank)).astype(np.float32) * scale
    for b in range(w.B):
        hp = hot_pages(w, layer, b)
        if hp.size:
            c[b][:, hp, :, 0] += np.float32(2.0)
        tok = np.arange(w.Np * w.P).reshape(w.Np, w.P)
        c[b][:, tok >= lens[b]] = 0.0
    return basis, mean, bf16_bits(c)


# ---------------------------------------------------------------- whole pools

def _threads():
    return max(1, min(16, os.cpu_count() or 1))


def fill_pools(w: Workload, layer: int, k_pool, v_pool, bt=None, threads=None):
    """Write every row's keys/values (uint16 bits) into pools [n_phys, Hkv, P, d].

    Either pool may be None.  Rows are generated in parallel threads (numpy
    releases the GIL while drawing)."""
    if bt is None:
        bt = block_table(w, layer)

    def job(bg):
        b, g = bg
        if k_pool is not None:
            k_pool[bt[b], g] = to_bits(row_keys(w, layer, b, g), w.dtype).reshape(w.Np, w.P, w.d)
        if v_pool is not None:
            v_pool[bt[b], g] = to_bits(row_values(w, layer, b, g), w.dtype).reshape(w.Np, w.P, w.d)

    rows = [(b, g) for b in range(w.B) for g in range(w.Hkv)]
    with cf.ThreadPoolExecutor(threads or _threads()) as ex:
        list(ex.map(job, rows))


def query_tensor(w: Workload, layer: int = 0, qidx: int = 0):
    """(B, Hq, d) uint16 bits of every query head."""
    q = np.empty((w.B, w.Hq, w.d), dtype=np.uint16)
    for b in range(w.B):
        for g in range(w.Hkv):
            q[b, g * w.G:(g + 1) * w.G] = to_bits(queries(w, layer, b, g, qidx), w.dtype)
    return q
