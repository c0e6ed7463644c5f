"""Hot-buffer admission for a host-resident value pool (test infrastructure only).

AMASS (amass-kv 0.1.1 project page), "What is in the box" item 2 and the
AMASS-mem variant: the value cache lives in pinned, device-mapped host memory
with a bounded resident hot buffer plus a staging pool, and only the pages a
step actually calls stay in device memory.  Readings taken here (the page
leaves them open):

  * the buffer's unit is one (physical page, KV head), u = phys * Hkv + g:
    the P x d values one row's attention reads of a page.  A KV head's
    selection then needs room only for what that head called, so a buffer of
    a tenth of the units holds a step whose rows each keep a tenth of their
    pages (with whole pages as the unit, the union over the heads does not
    fit);
  * admission runs once per decode step after its selection and before its
    attention, so the attention reads every admitted unit from device memory
    and a called unit crosses the host link at most once;
  * the replacement rule is plain LRU over buffer slots:

  state:  slot_page[s]  unit held by slot s, or -1
          slot_stamp[s] step at which slot s was last used (0 = never)
          hot[u]        slot holding unit u, or -1
  step t with selected units U (every row's selection mapped through the
  block table to u = phys * Hkv + g, duplicates removed):
    1. every unit of U that is hot has its slot stamped t;
    2. the units of U that are not hot, ascending by unit id, are admitted
       into the slots with the smallest (stamp, slot index) among slots whose
       stamp is below t, one unit per slot, paired in ascending order of slot
       index with the units in ascending order; if there are fewer such slots
       than units, the lowest unit ids are admitted;
    3. an admitted slot drops its old unit (hot[old] = -1), takes the new one
       and is stamped t; its V data is copied from the host pool.

HotBuffer is the same for any integer ids (pages or units).

Pinned in tests/test_oracle_hotbuffer.py: hand-worked sequences (fill, hit,
eviction of the least recently used, ties by slot index, more misses than free
slots), invariants over seeded random sequences (hot and slot_page are inverse
maps, no more than n_slots ids hot, every id of the step hot when it fits),
and the units of a hand-worked selection.
"""

import numpy as np


class HotBuffer:
    def __init__(self, n_ids, n_slots):
        self.slot_page = np.full(n_slots, -1, dtype=np.int64)
        self.slot_stamp = np.zeros(n_slots, dtype=np.int64)
        self.hot = np.full(n_ids, -1, dtype=np.int64)

    def step(self, pages, t):
        """Apply one step's admission; returns the (id, slot) copies, in slot order."""
        U = np.unique(np.asarray(pages, dtype=np.int64))
        hit = self.hot[U] >= 0
        self.slot_stamp[self.hot[U[hit]]] = t
        miss = U[~hit]                                   # ascending
        free = np.nonzero(self.slot_stamp < t)[0]
        order = np.lexsort((free, self.slot_stamp[free]))   # (stamp, slot) ascending
        n = min(miss.size, free.size)
        victims = np.sort(free[order[:n]])
        admit = miss[:n]
        copies = []
        for p, s in zip(admit, victims):
            old = self.slot_page[s]
            if old >= 0:
                self.hot[old] = -1
            self.slot_page[s] = p
            self.hot[p] = s
            self.slot_stamp[s] = t
            copies.append((int(p), int(s)))
        return copies


def selected_physical_pages(sel, sel_count, block_table, Hkv, seq_lens, page_size):
    """Physical pages a step selected and attention reads: entries i < sel_count
    (clamped to [0, k_max]) of sel [B, Hkv, k_max] with 0 <= p < Np_b."""
    out = []
    B, max_pages = block_table.shape
    k_max = sel.shape[-1]
    for b in range(B):
        npg = min(max_pages, -(-int(seq_lens[b]) // page_size)) if seq_lens[b] > 0 else 0
        for g in range(Hkv):
            k = min(max(int(sel_count[b, g]), 0), k_max)
            lp = np.asarray(sel[b, g, :k], dtype=np.int64)
            lp = lp[(lp >= 0) & (lp < npg)]
            out.append(block_table[b, lp])
    return np.unique(np.concatenate(out)) if out else np.zeros(0, np.int64)


def selected_units(sel, sel_count, block_table, Hkv, seq_lens, page_size):
    """Units u = phys * Hkv + g a step's attention reads: entries i < sel_count
    (clamped to [0, k_max]) of row (b, g) of sel [B, Hkv, k_max] with
    0 <= p < Np_b, through the block table; duplicates removed, ascending."""
    out = []
    B, max_pages = block_table.shape
    k_max = sel.shape[-1]
    for b in range(B):
        npg = min(max_pages, -(-int(seq_lens[b]) // page_size)) if seq_lens[b] > 0 else 0
        for g in range(Hkv):
            k = min(max(int(sel_count[b, g]), 0), k_max)
            lp = np.asarray(sel[b, g, :k], dtype=np.int64)
            lp = lp[(lp >= 0) & (lp < npg)]
            out.append(block_table[b, lp].astype(np.int64) * Hkv + g)
    return np.unique(np.concatenate(out)) if out else np.zeros(0, np.int64)
