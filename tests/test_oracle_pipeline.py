"""Oracle decode step on the seeded workloads (CPU only).

A sanity check, not parity: on the tiny workload (4 planted high-mass pages per
sequence, keys = 3 u_g + noise) the oracle's top-8 pages per KV head contain
every planted page, with per-page summaries and with the shared-basis ones; the
generator reproduces any row on its own; and the drifting-query recipe of the
host-resident runs has the stated statistics.
"""

import numpy as np

from oracle.pipeline import decode_row
from quantized_kv_cache_summary_amd import workloads as wl


def test_planted_pages_are_selected_tiny():
    w = wl.WORKLOADS["tiny"]
    for b in range(w.B):
        hp = set(wl.hot_pages(w, 0, b).tolist())
        assert len(hp) == 4
        for g in range(w.Hkv):
            q = wl.queries(w, 0, b, g)
            K = wl.row_keys(w, 0, b, g)
            V = wl.row_values(w, 0, b, g)
            r = decode_row(q, K, V, w.ctx, w.P, w.rank, w.tau, k_fixed=w.k_fixed)
            assert r["k"] == 8
            assert hp <= set(r["sel"].tolist())
            assert abs(np.exp(r["S"]).sum() - 1) < 1e-12


def test_planted_pages_are_selected_tiny_shared_basis():
    w = wl.WORKLOADS["tiny"]
    for b in range(w.B):
        hp = set(wl.hot_pages(w, 0, b).tolist())
        for g in range(w.Hkv):
            q = wl.queries(w, 0, b, g)
            r = decode_row(q, wl.row_keys(w, 0, b, g), wl.row_values(w, 0, b, g), w.ctx, w.P, w.rank,
                           w.tau, k_fixed=w.k_fixed, shared_basis=True)
            assert hp <= set(r["sel"].tolist())
            assert abs(np.exp(r["S"]).sum() - 1) < 1e-12


def test_generator_rows_are_independent_and_repeatable():
    w = wl.WORKLOADS["llama8b_32k"].replace(ctx=1024, B=2)
    a = wl.row_keys(w, 0, 1, 3)
    b = wl.row_keys(w, 0, 1, 3)
    np.testing.assert_array_equal(a, b)
    c = wl.row_keys(w, 0, 1, 4)
    assert not np.array_equal(a, c)
    # values are exact bf16 numbers
    np.testing.assert_array_equal(wl.round16(a, "bf16"), a)
    bt = wl.block_table(w)
    assert sorted(bt.ravel().tolist()) == list(range(w.n_phys))
    kp = np.zeros((w.n_phys, w.Hkv, w.P, w.d), np.uint16)
    wl.fill_pools(w, 0, kp, None, threads=2)
    np.testing.assert_array_equal(wl.bits_to_f32(kp[bt[1], 3].reshape(-1, w.d), "bf16"), a)


def test_tier_assignment_fractions():
    w = wl.WORKLOADS["tiers_64k"].replace(ctx=16 * 1000, B=2)
    t = wl.page_tiers(w)
    for b in range(w.B):
        counts = np.bincount(t[b], minlength=5)
        assert list(counts) == [50, 150, 300, 400, 100]


def test_worked_step_closed_forms():
    """A whole step on a hand-worked row (tests/golden/worked_step.json):
    degenerate and one-token pages give exact scores, so the normalisers,
    group scores, the top-k set for k = 1, 2, 3 and every attention output are
    closed forms in e, derived by hand from the definitions."""
    import json
    import os
    fx = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "worked_step.json")))
    q = np.array(fx["q"])
    keys, values = np.array(fx["keys"]), np.array(fx["values"])
    s_ref = np.array(fx["s_hat"])
    for case in fx["cases"]:
        r = decode_row(q, keys, values, fx["seq_len"], fx["page_size"], fx["rank"], fx["tau"],
                       k_fixed=case["k_fixed"])
        # log n is stored in float32 (log 2 to 2e-9), everything else is exact
        np.testing.assert_allclose(r["s_hat"], s_ref, rtol=0, atol=1e-7)
        np.testing.assert_allclose(r["S"], fx["S"], rtol=0, atol=1e-7)
        assert r["k"] == case["k_fixed"]
        assert r["sel"].tolist() == case["sel"]
        np.testing.assert_allclose(r["out"], case["out"], rtol=0, atol=1e-7)
        np.testing.assert_allclose(r["lse"], case["lse"], rtol=0, atol=1e-7)
    # with every page selected the attention's lse is the score's normaliser L_h
    np.testing.assert_allclose(fx["cases"][2]["lse"], fx["L"], rtol=0, atol=1e-12)
    np.testing.assert_allclose(np.exp(fx["S"]), fx["masses"], rtol=1e-12)
    # coverage mode: the shortest prefix of the S order whose mass reaches the target
    for case in fx["coverage_cases"]:
        r = decode_row(q, keys, values, fx["seq_len"], fx["page_size"], fx["rank"], fx["tau"],
                       coverage=case["coverage"])
        assert r["k"] == case["k"] and r["sel"].tolist() == case["sel"], case


def test_drift_queries_recipe():
    """The host-resident runs' drifting queries: q_0 is query draw 0, every
    step keeps N(0, 1) marginals, and consecutive queries have cosine about c."""
    w = wl.WORKLOADS["heavy70b_128k"]
    c = 0.95
    q = wl.drift_queries(w, 0, 3, 5, 40, c).astype(np.float64)
    assert np.array_equal(q[0], wl.queries(w, 0, 3, 5, 0))
    cos = [float(np.sum(q[t] * q[t + 1]) / np.linalg.norm(q[t]) / np.linalg.norm(q[t + 1])) for t in range(39)]
    assert abs(np.mean(cos) - c) < 0.01
    assert abs(q.std() - 1.0) < 0.05
    iid = np.stack([wl.queries(w, 0, 3, 5, j) for j in range(2)]).astype(np.float64)
    assert abs(float(np.sum(iid[0] * iid[1]) / np.linalg.norm(iid[0]) / np.linalg.norm(iid[1]))) < 0.2
