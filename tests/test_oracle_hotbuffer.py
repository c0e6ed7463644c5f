"""Pins for the hot-buffer admission rule (CPU only): a hand-worked sequence and
invariants over seeded random sequences."""

import numpy as np

from oracle.hotbuffer import HotBuffer, selected_physical_pages, selected_units


def test_hand_worked_sequence():
    h = HotBuffer(n_ids=10, n_slots=3)
    assert h.step([5, 2, 5], 1) == [(2, 0), (5, 1)]                 # fill: free slots by index
    assert h.step([5, 7, 9], 2) == [(7, 0), (9, 2)]                 # 5 hits; LRU slot 2 (never) then 0
    assert list(h.hot[[2, 5, 7, 9]]) == [-1, 1, 0, 2]
    assert h.step([2], 3) == [(2, 0)]                               # equal stamps: lowest slot
    assert h.step([1, 3, 4, 6], 4) == [(1, 0), (3, 1), (4, 2)]     # more misses than slots
    assert h.hot[6] == -1 and list(h.slot_page) == [1, 3, 4] and list(h.slot_stamp) == [4, 4, 4]
    assert h.step([1, 3, 4, 6], 5) == []                            # no slot is older than step 5
    assert list(h.slot_stamp) == [5, 5, 5]


def test_invariants_random_sequences():
    rng = np.random.default_rng(5)
    for trial in range(200):
        n_phys = int(rng.integers(4, 60))
        n_slots = int(rng.integers(1, 20))
        h = HotBuffer(n_phys, n_slots)
        for t in range(1, 30):
            U = np.unique(rng.integers(0, n_phys, int(rng.integers(0, 2 * n_slots + 2))))
            before = h.hot.copy()
            copies = h.step(U, t)
            hot_pages = np.nonzero(h.hot >= 0)[0]
            assert hot_pages.size <= n_slots
            for p in hot_pages:
                assert h.slot_page[h.hot[p]] == p
            for s, p in enumerate(h.slot_page):
                assert p < 0 or h.hot[p] == s
            if U.size <= n_slots:
                assert np.all(h.hot[U] >= 0)                        # the whole step fits
            assert all(before[p] < 0 for p, _ in copies)            # only misses are copied
            assert sorted(s for _, s in copies) == [s for _, s in copies]


def test_selected_pages_follow_counts_and_lengths():
    bt = np.array([[7, 3, 5, 1], [0, 2, 4, 6]])
    sel = np.array([[[0, 2, 3, -1], [1, 3, 0, 0]], [[3, 1, 0, 0], [2, 0, 0, 0]]])
    cnt = np.array([[3, 2], [2, 9]])                                # 9 clamps to k_max = 4
    got = selected_physical_pages(sel, cnt, bt, 2, seq_lens=np.array([64, 30]), page_size=16)
    # row (0,0): pages 0,2,3 -> 7,5,1; row (0,1): 1,3 -> 3,1; sequence 1 has 2 pages:
    # row (1,0): 3 (skipped), 1 -> 2; row (1,1): 2 (skipped), 0,0,0 -> 0
    assert list(got) == [0, 1, 2, 3, 5, 7]


def test_selected_units_follow_counts_lengths_and_heads():
    bt = np.array([[7, 3, 5, 1], [0, 2, 4, 6]])
    sel = np.array([[[0, 2, 3, -1], [1, 3, 0, 0]], [[3, 1, 0, 0], [2, 0, 0, 0]]])
    cnt = np.array([[3, 2], [2, 9]])                                # 9 clamps to k_max = 4
    got = selected_units(sel, cnt, bt, 2, seq_lens=np.array([64, 30]), page_size=16)
    # u = phys * 2 + g.  Row (0,0): phys 7,5,1 -> 14,10,2; row (0,1): phys 3,1 -> 7,3;
    # row (1,0): page 3 past the 2 pages, page 1 -> phys 2 -> 4; row (1,1): pages 0,0,0 -> phys 0 -> 1
    assert list(got) == [1, 2, 3, 4, 7, 10, 14]
    # the same physical page selected by both heads is two units
    sel2 = np.array([[[1], [1]]])
    got2 = selected_units(sel2, np.array([[1, 1]]), np.array([[4, 9]]), 2, seq_lens=np.array([32]), page_size=16)
    assert list(got2) == [18, 19]
