"""Decode-attention throughput on one MI355X: steps/s and effective HBM bandwidth.

One step = kv_page_score + kv_page_topk + kv_sparse_decode_attn (+ its split
merge) for one decoder layer of the whole batch, inputs resident in HBM.  The
default workload is the Llama-3-8B-shaped decode layer at 32K context
(B=8, 32 query / 8 KV heads, d=128, bf16, page 16, rank 4, keep 8 %).  Several
independent layers are rotated so that the bytes touched between two visits of
one layer exceed the 256 MB last-level cache, and each step uses one of 16
pre-generated queries.

Prints one JSON line on stdout; progress goes to stderr.
"""

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "decode attn steps/sec & effective HBM GB/s (% peak) at 32k-128k ctx, 1 GPU"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default="llama8b_32k")
    ap.add_argument("--layers", type=int, default=0, help="rotated layers (0 = enough to exceed 4x256 MB)")
    ap.add_argument("--queries", type=int, default=16)
    ap.add_argument("--cpu-seconds", type=float, default=15.0, help="budget of the oracle baseline")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-basis", action="store_true",
                    help="skip the shared-basis summary variant (reported beside the headline)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of a HIP graph replay")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 512 MiB device copy (known bytes) for scaling counter readings")
    ap.add_argument("--groups", type=int, default=1,
                    help="row groups per step, each on its own stream (1 = one chain for the batch)")
    return ap.parse_args()


def algorithmic_bytes(w, sel_counts):
    rec = (1 + w.rank) * w.d * 2 + 4                       # bf16 record + float32 log n
    summary = w.rows * w.Np * rec
    selected = int(sel_counts.sum()) * w.P * w.d * 2 * 2   # K and V, 16-bit
    return summary, selected


def basis_algorithmic_bytes(w, sel_counts):
    rec = w.d * 2 + w.rank * 4 + 4                          # bf16 mean + float32 variances + log n
    summary = w.rows * w.Np * rec + w.rows * w.rank * w.d * 4   # + the float32 row bases
    selected = int(sel_counts.sum()) * w.P * w.d * 2 * 2
    return summary, selected


def traffic_for(workload):
    """HBM bytes per launch of the score kernel from the committed counter runs
    (profiles/), if they were taken on the current kernel source; else None."""
    from quantized_kv_cache_summary_amd import traffic
    path = os.path.join(ROOT, "profiles", f"page_score_{workload}_traffic.json")
    try:
        t = json.load(open(path))
    except (OSError, ValueError):
        return None
    if t.get("kernel_source_sha256") != traffic.score_kernel_hash():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, budget_s):
    """The oracle's decode step on a sample of rows, scaled to the whole batch."""
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(limits=1)
    except Exception:
        limiter = None
    import oracle
    from quantized_kv_cache_summary_amd import workloads as wl

    rows = []
    t_build = 0.0
    for g in range(min(4, w.Hkv)):
        q = wl.queries(w, 0, 0, g).astype(np.float64)
        K = wl.row_keys(w, 0, 0, g).astype(np.float64)[: w.ctx]
        V = wl.row_values(w, 0, 0, g).astype(np.float64)[: w.ctx]
        t0 = time.perf_counter()
        summ = oracle.pipeline.build_row_summaries(K, w.ctx, w.P, w.rank)
        t_build += time.perf_counter() - t0
        rows.append((q, K, V, summ))
    n_done = 0
    t0 = time.perf_counter()
    while True:
        for q, K, V, summ in rows:
            oracle.decode_row(q, K, V, w.ctx, w.P, w.rank, w.tau, w.keep, w.k_fixed, summary=summ)
            n_done += 1
        el = time.perf_counter() - t0
        if el >= budget_s or n_done >= 4000:
            break
    per_row = el / n_done
    if limiter is not None:
        limiter.unregister() if hasattr(limiter, "unregister") else None
    return {
        "value": 1.0 / (per_row * w.rows), "unit": "steps/s", "cores": 1, "kind": "oracle",
        "sample": (f"{n_done} oracle row-steps (score, group aggregate, top-k, sparse attention; float64, "
                   f"summaries prebuilt in {t_build:.1f}s untimed) over {len(rows)} of {w.rows} rows of "
                   f"{w.name}; {per_row * 1e3:.2f} ms per row, scaled x{w.rows} to one full-batch step; "
                   f"BLAS limited to 1 thread"),
    }


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    from quantized_kv_cache_summary_amd import harness as hz
    from quantized_kv_cache_summary_amd import kvsparse as kv
    from quantized_kv_cache_summary_amd import workloads as wl

    w = wl.WORKLOADS[args.workload]
    if w.v_host or w.tier_fracs is not None:
        raise SystemExit("bench.py times the resident native-tier workloads; see the tests for the others")
    torch.cuda.set_device(0)
    # bytes one step touches: every summary record plus the selected K/V pages
    touched = w.rows * w.Np * ((1 + w.rank) * w.d * 2 + 4) + w.rows * w.k_of(w.Np) * w.P * w.d * 2 * 2
    n_layers = args.layers or max(1, math.ceil(4 * 256e6 / touched))
    log(f"[bench] workload {w.name}: {n_layers} layers rotated, {touched / 1e6:.1f} MB touched per step, "
        f"{args.queries} queries")
    t0 = time.time()
    layers = [hz.DeviceLayer(w, layer=i, summaries="build") for i in range(n_layers)]
    qs = [[hz.queries_device(w, i, j) for j in range(args.queries)] for i in range(n_layers)]
    bufs = [hz.StepBuffers(w) for _ in range(n_layers)]
    steps_split = [hz.SplitStep(layers[i], bufs[i], args.groups) for i in range(n_layers)]
    torch.cuda.synchronize()
    log(f"[bench] set-up {time.time() - t0:.1f}s (generation, upload, summary build)")

    stream = torch.cuda.current_stream()

    def step(i):
        li = i % n_layers
        q = qs[li][(i // n_layers) % args.queries]
        steps_split[li](q)

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 x 512 MiB device-to-device copies")

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    log(f"[bench] warmup {args.warmup} steps done")

    # ---- eager single chain (context only)
    K = args.steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for i in range(K):
        li = i % n_layers
        q = qs[li][(i // n_layers) % args.queries]
        hz.score(layers[li], q, bufs[li])
        hz.topk(layers[li], bufs[li])
        hz.attend(layers[li], q, bufs[li])
    e1.record(stream)
    torch.cuda.synchronize()
    eager_ms = e0.elapsed_time(e1) / K

    # ---- per-kernel averages: back-to-back launches of one kernel over the
    #      rotated layers, replayed from a HIP graph, HIP events on the launch
    #      stream around the replays; average launch duration = elapsed /
    #      launches.  The score kernel's figure is the roofline's.
    def graph_avg_us(launch):
        n = n_layers * min(args.queries, 4)
        gk = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gk):
            for i in range(n):
                launch(i % n_layers, qs[i % n_layers][(i // n_layers) % args.queries])
        for _ in range(3):
            gk.replay()
        torch.cuda.synchronize()
        reps = max(1, K // n)
        k0, k1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        k0.record(stream)
        for _ in range(reps):
            gk.replay()
        k1.record(stream)
        torch.cuda.synchronize()
        return k0.elapsed_time(k1) * 1e3 / (reps * n), reps * n

    score_us, n_score = graph_avg_us(lambda li, q: hz.score(layers[li], q, bufs[li]))
    topk_us, _ = graph_avg_us(lambda li, q: hz.topk(layers[li], bufs[li]))
    attend_us, _ = graph_avg_us(lambda li, q: hz.attend(layers[li], q, bufs[li]))
    score_ms = np.array([score_us / 1e3])
    log(f"[bench] eager single chain: {eager_ms * 1e3:.1f} us/step; per launch: score {score_us:.2f} us "
        f"({n_score} graph-replayed launches), top-k {topk_us:.2f} us, attention {attend_us:.2f} us")

    # ---- timed region: K steps (row groups overlapped on streams), replayed
    #      from a HIP graph that holds one pass over the rotated layers
    if args.eager:
        timed_steps = K
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(K):
            step(i)
        b.record(stream)
        torch.cuda.synchronize()
        ms_per_step = a.elapsed_time(b) / K
    else:
        n_cap = n_layers * min(args.queries, 4)     # every layer with 4 different queries
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n_cap):
                step(i)
        for _ in range(3):
            g.replay()
        torch.cuda.synchronize()
        reps = max(1, K // n_cap)
        timed_steps = reps * n_cap
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
        ms_per_step = a.elapsed_time(b) / timed_steps
    log(f"[bench] timed {timed_steps} steps: {ms_per_step * 1e3:.1f} us/step")

    sel_counts = bufs[0].sel_count.cpu().numpy()
    summary_b, selected_b = algorithmic_bytes(w, sel_counts)
    step_bytes = summary_b + selected_b
    score_avg_s = float(score_ms.mean()) / 1e3
    achieved = summary_b / score_avg_s / 1e9
    best_ms = ms_per_step
    result = {
        "metric": METRIC,
        "value": 1e3 / best_ms,
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": timed_steps,
        "warmup": args.warmup,
        "ms_per_step": best_ms,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys/values with planted hot pages and a sink page; no dataset)",
        "config": {
            "workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
            "page_size": w.P, "ctx": w.ctx, "rank": w.rank, "keep": w.keep, "k_per_row": int(sel_counts.max()),
            "rotated_layers": n_layers, "row_groups_on_streams": args.groups,
            "timing": "eager" if args.eager else "hip graph replay",
        },
        "effective_GBps": step_bytes / (best_ms / 1e3) / 1e9,
        "pct_hbm_peak": 100.0 * step_bytes / (best_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": {"summaries": summary_b, "selected_kv": selected_b},
        "eager_single_chain_ms_per_step": eager_ms,
        "kernel_avg_us": {"page_score": score_us, "page_topk": topk_us, "sparse_decode_attn": attend_us},
        "roofline": {
            "kernel": "page_score_kernel",
            "bound": "hbm",
            "achieved": achieved,
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS,
            "traffic": traffic_for(w.name),
            "avg_launch_us": score_avg_s * 1e6,
            "bytes_per_launch": summary_b,
        },
    }
    if not args.no_basis:
        # the same layers scored from shared-basis summaries (row basis built
        # from each layer's keys, then per-page means and variances), same
        # rotation, queries, selection rule, attention and timing
        t0 = time.time()
        blayers = [l.with_basis_summaries() for l in layers]
        torch.cuda.synchronize()
        log(f"[bench] shared-basis summaries built in {time.time() - t0:.1f}s")
        bsteps = [hz.SplitStep(blayers[i], bufs[i], 1) for i in range(n_layers)]
        n_cap = n_layers * min(args.queries, 4)
        for i in range(args.warmup):
            bsteps[i % n_layers](qs[i % n_layers][(i // n_layers) % args.queries])
        gb = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gb):
            for i in range(n_cap):
                bsteps[i % n_layers](qs[i % n_layers][(i // n_layers) % args.queries])
        for _ in range(3):
            gb.replay()
        torch.cuda.synchronize()
        reps = max(1, K // n_cap)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            gb.replay()
        b.record(stream)
        torch.cuda.synchronize()
        b_ms = a.elapsed_time(b) / (reps * n_cap)
        bscore_us, _ = graph_avg_us(lambda li, q: hz.score(blayers[li], q, bufs[li]))
        bsel = bufs[0].sel_count.cpu().numpy()
        bsum, bselb = basis_algorithmic_bytes(w, bsel)
        log(f"[bench] shared-basis step {b_ms * 1e3:.1f} us, score {bscore_us:.2f} us")
        result["shared_basis"] = {
            "value": 1e3 / b_ms, "unit": "steps/s", "ms_per_step": b_ms, "steps": reps * n_cap,
            "effective_GBps": (bsum + bselb) / (b_ms / 1e3) / 1e9,
            "pct_hbm_peak": 100.0 * (bsum + bselb) / (b_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
            "algorithmic_bytes_per_step": {"summaries": bsum, "selected_kv": bselb},
            "score_kernel": {"avg_launch_us": bscore_us, "achieved_GBps": bsum / (bscore_us * 1e3),
                             "frac": bsum / (bscore_us * 1e3) / HBM_PEAK_GBS},
            "note": "same layers, queries and attention; summaries = shared row basis + per-page mean "
                    "and variances (not the headline's per-page directions)",
        }
    # coverage-mode selection (k per row from the mass prefix) on the headline
    # layers' scores: its kernel time and the k it picks, for context
    from quantized_kv_cache_summary_amd import kvsparse as kvs
    cov_sel = [torch.empty((w.B, w.Hkv, w.Np), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
    cov_cnt = [torch.empty((w.B, w.Hkv), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
    for li in range(n_layers):
        hz.score(layers[li], qs[li][0], bufs[li])
    cov = {}
    for c in (0.5, 0.95):
        us, _ = graph_avg_us(lambda li, q: kvs.page_topk_coverage(layers[li].L, bufs[li].head_scores,
                                                                  bufs[li].lse_partial, layers[li].seq_lens, w.Np,
                                                                  c, cov_sel[li], cov_cnt[li]))
        kk = cov_cnt[0].cpu().numpy()
        cov[str(c)] = {"avg_launch_us": us, "k_mean": float(kk.mean()), "k_min": int(kk.min()),
                       "k_max": int(kk.max())}
    result["coverage_topk"] = cov
    log(f"[bench] coverage-mode top-k: {cov}")
    if not args.no_cpu_baseline:
        log("[bench] oracle baseline on the host ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    for l in layers:
        l.release()
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
