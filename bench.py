"""Decode-attention throughput on one MI355X: steps/s and effective HBM bandwidth.

One step = kv_page_score + kv_page_topk + kv_sparse_decode_attn (+ its split
merge) for one decoder layer of the whole batch, inputs resident in HBM, issued
by one kv_sparse_decode_step call (which fuses top-k into the attention launch
where that is the faster schedule).  The headline workload is the
Llama-3-8B-shaped decode layer at 32K context (B=8, 32 query / 8 KV heads,
d=128, bf16, page 16, rank 4, keep 8 %).  Several independent layers are rotated
so that the bytes touched between two visits of one layer exceed the 256 MB
last-level cache, and each step uses one of a few pre-generated queries.

The default run also measures the other long-context workloads the same way
(mixed-precision tiers at 64K, the Qwen2.5-3B shape at 128K, the 70B shape at
128K with K and V in HBM, and that shape with V in pinned host memory behind a
hot buffer) and reports each under "configs".

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
HEADLINE = "llama8b_32k"
# the other workloads of the metric's 32K-128K range, measured in the default run
OTHER_CONFIGS = ("tiers_64k", "qwen3b_128k", "heavy70b_128k_v_in_hbm", "heavy70b_128k_host_v")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", default=HEADLINE)
    ap.add_argument("--configs", default="auto",
                    help="comma-separated other workloads to measure beside the headline, 'none', or 'auto' "
                         "(all of them when the headline workload is the default one)")
    ap.add_argument("--layers", type=int, default=0, help="rotated layers (0 = enough to exceed 4x256 MB)")
    ap.add_argument("--queries", type=int, default=4)
    ap.add_argument("--cpu-seconds", type=float, default=6.0, help="budget of each oracle baseline run")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-basis", action="store_true",
                    help="skip the shared-basis and r8 summary variants (reported beside the headline)")
    ap.add_argument("--eager", action="store_true", help="time eager launches instead of HIP graph replays")
    ap.add_argument("--no-extras", action="store_true",
                    help="skip the context lines (dense attention, coverage-mode top-k, ...), e.g. under a profiler")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="also run a 512 MiB device copy (known bytes) for scaling counter readings")
    ap.add_argument("--mem-kv", action="store_true",
                    help="host-resident workloads: also time the variant with K in host memory too")
    ap.add_argument("--two-kernel", action="store_true",
                    help="time the step as separate top-k and attention launches (default: the fused call "
                         "where it is the faster step)")
    ap.add_argument("--splits", type=int, default=0, help="attention splits per row (0 = the library's choice)")
    ap.add_argument("--groups", type=int, default=1,
                    help="row groups per step, each on its own stream (1 = one chain for the batch)")
    return ap.parse_args()


TIER_BITS = {0: 16, 1: 8, 2: 4, 3: 2, 4: 1, 5: 8}


def page_bytes(w, tier):
    """K plus V bytes of one (row, page) in a tier: codes plus a 4-byte
    (scale, zero) pair per 32-element group for the packed tiers."""
    if tier == 0:
        return 2 * w.P * w.d * 2
    return 2 * w.P * (w.d * TIER_BITS[tier] // 8 + (w.d // 32) * 4)


def record_bytes(w):
    return (1 + w.rank) * w.d * 2 + 4                       # bf16 record + float32 log n


def algorithmic_bytes(w, sel_counts, sel=None, tiers=None):
    """Summary bytes and selected K/V bytes of one step; with tiers (B, Np) the
    selected pages are priced at their tier's size (sel gives the pages)."""
    import numpy as np
    summary = w.rows * w.Np * record_bytes(w)
    if tiers is None:
        return summary, int(sel_counts.sum()) * page_bytes(w, 0)
    selected = 0
    for b in range(w.B):
        for g in range(w.Hkv):
            pages = sel[b, g, :sel_counts[b, g]]
            for t, n in zip(*np.unique(tiers[b, pages], return_counts=True)):
                selected += int(n) * page_bytes(w, int(t))
    return summary, selected


def basis_algorithmic_bytes(w, sel_counts):
    rec = w.d * 2 + w.rank * 4 + 4                          # bf16 mean + float32 variances + log n
    summary = w.rows * w.Np * rec + w.rows * w.rank * w.d * 4   # + the float32 row bases
    selected = int(sel_counts.sum()) * w.P * w.d * 2 * 2
    return summary, selected


def _gm(G):
    return 4 if G <= 4 else (8 if G <= 8 else 16)


def step_kernels(w, fused, tiered):
    """rocprofv3 names of the kernels one step launches, by role."""
    f16 = "true" if w.dtype == "f16" else "false"
    gm = _gm(w.G)
    names = {"score": f"kvs::page_score_kernel<{w.d}, {w.rank}, {f16}>"}
    t = "true" if tiered else "false"
    if fused:
        names["topk_attention"] = f"kvs::sparse_attn_kernel<{w.d}, {gm}, {f16}, {t}, true>"
    else:
        names["topk"] = f"kvs::page_topk_kernel<{gm}, {1024 if w.Np >= 4096 else 512}>"
        names["attention"] = f"kvs::sparse_attn_kernel<{w.d}, {gm}, {f16}, {t}, false>"
    return names


def traffic_for(workload, kernel):
    """HBM bytes (read + written) per launch of `kernel` from the committed
    counter runs (profiles/traffic_<workload>.json), if they were taken on the
    kernel's current sources; else None."""
    from quantized_kv_cache_summary_amd import traffic
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    try:
        t = json.load(open(path))["kernels"][kernel]
    except (OSError, ValueError, KeyError):
        return None
    if t.get("sources_sha256") != traffic.kernel_sources_hash(kernel):
        return None
    return t.get("hbm_bytes_per_launch")


def roofline_entry(name, nbytes, avg_us, workload, what):
    achieved = nbytes / (avg_us * 1e3)
    return {"kernel": name, "bound": "hbm", "achieved": achieved, "peak": HBM_PEAK_GBS, "unit": "GB/s",
            "frac": achieved / HBM_PEAK_GBS, "traffic": traffic_for(workload, name),
            "avg_launch_us": avg_us, "bytes_per_launch": nbytes, "algorithmic_bytes": what}


# ---------------------------------------------------------------- the oracle on the host

def _oracle_rows_worker(job):
    """One host process: the oracle's decode step on one row, repeated until the
    budget is spent (summaries built before the clock starts).  Runs in a
    spawned child that never touches the GPU."""
    name, b, g, budget_s, start_at = job
    for var in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS"):
        os.environ[var] = "1"
    import numpy as np
    try:
        from threadpoolctl import threadpool_limits
        threadpool_limits(limits=1)       # after numpy has loaded its BLAS
    except Exception:
        pass
    import oracle
    from quantized_kv_cache_summary_amd import workloads as wl
    w = wl.WORKLOADS[name]
    q = wl.queries(w, 0, b, g).astype(np.float64)
    K = wl.row_keys(w, 0, b, g).astype(np.float64)[: w.ctx]
    V = wl.row_values(w, 0, b, g).astype(np.float64)[: w.ctx]
    summ = oracle.pipeline.build_row_summaries(K, w.ctx, w.P, w.rank)
    while time.time() < start_at:
        time.sleep(0.01)
    n = 0
    t0 = time.perf_counter()
    while True:
        oracle.decode_row(q, K, V, w.ctx, w.P, w.rank, w.tau, w.keep, w.k_fixed, summary=summ)
        n += 1
        el = time.perf_counter() - t0
        if el >= budget_s:
            return n, el


def cpu_baseline(w, budget_s):
    """The oracle's decode step (score, group aggregate, top-k, sparse attention;
    float64) on the host: one process per core over distinct rows, and one
    thread alone; both scaled to one full-batch step."""
    import concurrent.futures as cf
    import multiprocessing as mp
    import numpy as np
    try:
        from threadpoolctl import threadpool_info
        blas = [(i.get("internal_api"), i.get("num_threads")) for i in threadpool_info()]
    except Exception:
        blas = None
    n_cpu = os.cpu_count() or 1
    workers = max(1, min(16, n_cpu, w.rows))
    rows = [(b, g) for b in range(w.B) for g in range(w.Hkv)][:workers]
    start_at = time.time() + 6.0 + w.ctx / 32768 * 2.0     # summaries are built before this
    with cf.ProcessPoolExecutor(workers, mp_context=mp.get_context("spawn")) as ex:
        res = list(ex.map(_oracle_rows_worker, [(w.name, b, g, budget_s, start_at) for b, g in rows]))
    rows_per_s = sum(n / el for n, el in res)
    # one thread alone (this process, BLAS limited to one thread)
    one = _oracle_rows_worker((w.name, 0, 0, budget_s, 0.0))
    one_rows_per_s = one[0] / one[1]
    return {
        "value": rows_per_s / w.rows, "unit": "steps/s", "cores": workers, "kind": "oracle",
        "sample": (f"{sum(n for n, _ in res)} oracle row-steps in {budget_s:.0f}s on {workers} processes "
                   f"(one row of {w.name} each, BLAS 1 thread per process, summaries prebuilt untimed); "
                   f"{rows_per_s:.1f} rows/s scaled to the {w.rows}-row step"),
        "host_cpu_count": n_cpu,
        "blas": blas,
        "one_thread": {"value": one_rows_per_s / w.rows, "unit": "steps/s", "cores": 1,
                       "ms_per_row": 1e3 / one_rows_per_s,
                       "sample": f"{one[0]} row-steps of row (0, 0) in {one[1]:.1f}s, one thread"},
    }


# ---------------------------------------------------------------- GPU timing helpers

def timed_region(step, n_layers, nq, K, stream, eager=False, dist_replays=8):
    """K steps, HIP events on the launch stream around them.  Graph mode: one
    graph holding a pass over every rotated layer with every query (n_layers x
    nq steps), replayed back to back with an event after every replay; the last
    replay holds the remainder, so exactly K steps are timed.  The per-step
    time of each full replay is a distribution sample; when K covers fewer than
    `dist_replays` full replays, further replays after the timed region add
    samples.  Returns (ms per step over the K timed steps, samples)."""
    import numpy as np
    import torch
    if eager:
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        a.record(stream)
        for i in range(K):
            step(i % n_layers, (i // n_layers) % nq)
        b.record(stream)
        torch.cuda.synchronize()
        return a.elapsed_time(b) / K, None
    n_cap = n_layers * nq

    def capture(n):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                step(i % n_layers, (i // n_layers) % nq)
        return g

    R = math.ceil(K / n_cap)
    last = K - (R - 1) * n_cap
    full_g = capture(n_cap)
    tail = full_g if last == n_cap else capture(last)
    for g in (full_g, tail):
        g.replay()
    torch.cuda.synchronize()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(R + 1)]
    ev[0].record(stream)
    for r in range(R):
        (full_g if r < R - 1 else tail).replay()
        ev[r + 1].record(stream)
    torch.cuda.synchronize()
    ms = ev[0].elapsed_time(ev[R]) / K
    full = R if last == n_cap else R - 1
    per = [ev[r].elapsed_time(ev[r + 1]) / n_cap for r in range(full)]
    extra = max(0, dist_replays - full)
    if extra:
        ex = [torch.cuda.Event(enable_timing=True) for _ in range(extra + 1)]
        ex[0].record(stream)
        for r in range(extra):
            full_g.replay()
            ex[r + 1].record(stream)
        torch.cuda.synchronize()
        per += [ex[r].elapsed_time(ex[r + 1]) / n_cap for r in range(extra)]
    return ms, np.array(per)


def graph_avg_us(launch, n_layers, nq, K, stream):
    """Average duration of one kernel: back-to-back launches over the rotated
    layers (and queries) captured in a HIP graph, replayed between HIP events on
    the launch stream; elapsed / launches."""
    import torch
    n = n_layers * nq
    gk = torch.cuda.CUDAGraph()
    with torch.cuda.graph(gk):
        for i in range(n):
            launch(i % n_layers, (i // n_layers) % nq)
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


def distribution(per):
    import numpy as np
    if per is None or len(per) == 0:
        return None
    return {"over": f"{len(per)} graph replays of one pass over every rotated layer and query (per-step time "
                    f"of each replay)",
            "median": float(np.median(per)), "p10": float(np.percentile(per, 10)),
            "p90": float(np.percentile(per, 90)), "min": float(np.min(per)), "max": float(np.max(per))}


# ---------------------------------------------------------------- one workload's step

def measure_step(w, args, extras, label=None):
    """Times the whole-batch decode step of workload w (inputs in HBM) and its
    kernels.  Returns the result dict (without the metric header) and the
    layers' state needed by the headline's extras."""
    import numpy as np
    import torch
    from quantized_kv_cache_summary_amd import harness as hz
    from quantized_kv_cache_summary_amd import kvsparse as kv
    from quantized_kv_cache_summary_amd import workloads as wl

    label = label or w.name
    tiers = wl.page_tiers(w)
    avg_page = (page_bytes(w, 0) if tiers is None else
                sum(f * page_bytes(w, t) for f, t in zip(w.tier_fracs, w.tier_order)))
    touched = w.rows * w.Np * record_bytes(w) + w.rows * w.k_of(w.Np) * avg_page
    n_layers = args.layers or max(1, math.ceil(4 * 256e6 / touched))
    nq = max(1, min(args.queries, 4))
    log(f"[bench] {label}: {n_layers} layers rotated, {touched / 1e6:.1f} MB touched per step, {nq} queries")
    t0 = time.time()
    layers = [hz.DeviceLayer(w, layer=i, summaries="build") for i in range(n_layers)]
    qs = [[hz.queries_device(w, i, j) for j in range(nq)] for i in range(n_layers)]
    bufs = [hz.StepBuffers(w, num_splits=args.splits) for _ in range(n_layers)]
    fused = not args.two_kernel and args.groups == 1 and hz.fused_preferred(layers[0], bufs[0])
    whole = not args.two_kernel and args.groups == 1 and hz.step_supported(layers[0], bufs[0])
    if whole:
        assert kv.step_fused(layers[0].L, layers[0].pages, w.B, w.Np, bufs[0].sel.shape[-1], args.splits) == fused
    steps_split = [hz.SplitStep(layers[i], bufs[i], args.groups, num_splits=args.splits, fused=fused)
                   for i in range(n_layers)]
    torch.cuda.synchronize()
    log(f"[bench] {label}: set-up {time.time() - t0:.1f}s (generation, upload, summary build)")
    stream = torch.cuda.current_stream()

    def step(li, j):
        if whole:
            hz.whole_step(layers[li], qs[li][j], bufs[li])
        else:
            steps_split[li](qs[li][j])

    if args.copy_calibration:
        src = torch.empty(512 << 20, dtype=torch.uint8, device="cuda").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst
        log("[bench] copy calibration: 3 x 512 MiB device-to-device copies")

    for i in range(args.warmup):
        step(i % n_layers, (i // n_layers) % nq)
    torch.cuda.synchronize()
    K = args.steps
    ms_per_step, per = timed_region(step, n_layers, nq, K, stream, eager=args.eager)
    log(f"[bench] {label}: timed {K} steps: {ms_per_step * 1e3:.1f} us/step"
        + (" (top-k and attention fused)" if fused else ""))

    # per-kernel averages of the kernels the step launches
    kn = step_kernels(w, fused, tiers is not None)
    kus = {"score": graph_avg_us(lambda li, j: hz.score(layers[li], qs[li][j], bufs[li]), n_layers, nq, K, stream)[0]}
    if fused:
        kus["topk_attention"] = graph_avg_us(lambda li, j: hz.topk_attend(layers[li], qs[li][j], bufs[li]),
                                             n_layers, nq, K, stream)[0]
    else:
        kus["topk"] = graph_avg_us(lambda li, j: hz.topk(layers[li], bufs[li]), n_layers, nq, K, stream)[0]
        kus["attention"] = graph_avg_us(lambda li, j: hz.attend(layers[li], qs[li][j], bufs[li]),
                                        n_layers, nq, K, stream)[0]
    # the selection of the last step (every layer selects the same count)
    hz.decode_step(layers[0], qs[0][0], bufs[0], fused=fused)
    torch.cuda.synchronize()
    sel_counts = bufs[0].sel_count.cpu().numpy()
    summary_b, selected_b = algorithmic_bytes(w, sel_counts, bufs[0].sel.cpu().numpy(), tiers)
    head_scores_b = w.rows * w.G * w.Np * 4
    step_bytes = summary_b + selected_b
    kbytes = {"score": (summary_b, "summary records (bf16 mean and directions, float32 log n)"),
              "topk": (head_scores_b, "head scores read once"),
              "attention": (selected_b, "K and V of the selected pages (codes and scale/zero for packed tiers)"),
              "topk_attention": (selected_b + head_scores_b,
                                 "K and V of the selected pages plus the head scores read once per row")}
    kernels = {role: roofline_entry(kn[role], kbytes[role][0], us, label, kbytes[role][1])
               for role, us in kus.items()}
    dominant = max(kernels, key=lambda r: kernels[r]["avg_launch_us"])
    roofline = dict(kernels[dominant])
    roofline["role"] = dominant
    roofline["kernels"] = kernels
    log(f"[bench] {label}: per launch " + ", ".join(f"{r} {e['avg_launch_us']:.2f} us ({e['frac'] * 100:.1f} %)"
                                                   for r, e in kernels.items()))
    res = {
        "value": 1e3 / ms_per_step, "unit": "steps/s", "ms_per_step": ms_per_step, "steps": K,
        "effective_GBps": step_bytes / (ms_per_step / 1e3) / 1e9,
        "pct_hbm_peak": 100.0 * step_bytes / (ms_per_step / 1e3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": {"summaries": summary_b, "selected_kv": selected_b},
        "step_ms_distribution": distribution(per),
        "config": {
            "workload": label, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
            "page_size": w.P, "ctx": w.ctx, "rank": w.rank, "keep": w.keep, "k_per_row": int(sel_counts.max()),
            "tiers": None if tiers is None else dict(zip([wl.TIER_NAMES[t] for t in w.tier_order], w.tier_fracs)),
            "rotated_layers": n_layers, "queries": nq, "row_groups_on_streams": args.groups,
            "step_call": "kv_sparse_decode_step" if whole else "separate calls",
            "topk_attention": "fused (kv_topk_sparse_decode_attn)" if fused else "separate launches",
            "timing": "eager" if args.eager else "hip graph replay",
        },
        "roofline": roofline,
    }
    state = dict(layers=layers, qs=qs, bufs=bufs, fused=fused, n_layers=n_layers, nq=nq, stream=stream,
                 sel_counts=sel_counts, tiers=tiers)
    return res, state


def release(state):
    import torch
    for l in state["layers"]:
        l.release()
    state.clear()
    torch.cuda.synchronize()
    torch.cuda.empty_cache()


def append_summary_build(w, args, st):
    """Append-time summary build, for context (not in the step): the newest
    page of every sequence rebuilt from its keys, one call per layer.  The
    rebuild writes the same record, so the layers are unchanged."""
    import numpy as np
    import torch
    from quantized_kv_cache_summary_amd import kvsparse as kv
    layers = st["layers"]
    if layers[0].summary is None or layers[0].seq_lens_np.min() < 1:
        return None
    last = (layers[0].seq_lens_np - 1) // w.P
    ent = torch.from_numpy(np.stack([np.arange(w.B), last], 1).astype(np.int32)).cuda()
    nval = torch.from_numpy((layers[0].seq_lens_np - last * w.P).astype(np.int32)).cuda()
    sb_us = graph_avg_us(lambda li, j: kv.summary_build(layers[li].L, layers[li].k_src, layers[li].bt, ent, nval,
                                                        layers[li].summary, layers[li].log_n),
                         st["n_layers"], st["nq"], args.steps, st["stream"])[0]
    log(f"[bench] append-time summary build ({w.B * w.Hkv} page-heads, P = {w.P}, rank {w.rank}): "
        f"{sb_us:.1f} us per call, {sb_us / w.P:.2f} us per step amortised")
    return {"avg_launch_us": sb_us, "page_heads": w.B * w.Hkv, "page_size": w.P, "rank": w.rank,
            "amortized_us_per_step": sb_us / w.P,
            "note": "kv_summary_build of the newest page of every sequence (one page per sequence per P "
                    "decode steps); append-time work, not in the timed step"}


def headline_extras(w, args, res, st):
    """Context lines of the headline workload (not part of the step)."""
    import numpy as np
    import torch
    from quantized_kv_cache_summary_amd import harness as hz
    from quantized_kv_cache_summary_amd import kvsparse as kv
    from quantized_kv_cache_summary_amd import workloads as wl
    layers, qs, bufs, fused = st["layers"], st["qs"], st["bufs"], st["fused"]
    n_layers, nq, stream, tiers = st["n_layers"], st["nq"], st["stream"], st["tiers"]
    K = args.steps

    def gavg(launch):
        return graph_avg_us(launch, n_layers, nq, K, stream)[0]

    if fused and not args.eager:
        # the same steps with separate top-k and attention launches
        two = [hz.SplitStep(layers[i], bufs[i], 1, num_splits=args.splits) for i in range(n_layers)]
        two_ms, _ = timed_region(lambda li, j: two[li](qs[li][j]), n_layers, nq, K, stream)
        res["two_kernel_step"] = {"ms_per_step": two_ms, "value": 1e3 / two_ms, "unit": "steps/s",
                                  "page_topk_avg_us": gavg(lambda li, j: hz.topk(layers[li], bufs[li])),
                                  "sparse_decode_attn_avg_us": gavg(lambda li, j: hz.attend(layers[li], qs[li][j],
                                                                                            bufs[li])),
                                  "note": "score, then kv_page_topk and kv_sparse_decode_attn as separate launches"}
        log(f"[bench] same steps with separate top-k and attention launches: {two_ms * 1e3:.1f} us/step")
    if tiers is not None:
        # attention alone over the same shape with every page in one packed
        # tier (same rotation, queries and selections): the decode cost per tier
        uni = {}
        sel_counts = st["sel_counts"]
        for t, outl in ((1, False), (5, False), (2, False), (3, False), (4, False), (4, True)):
            ulayers = [hz.DeviceLayer(w.replace(tier_fracs=(1.0,), tier_order=(t,)), layer=i, summaries=None,
                                      b1_outliers=outl) for i in range(n_layers)]
            us = gavg(lambda li, j: hz.attend(ulayers[li], qs[li][j], bufs[li]))
            b_sel = int(sel_counts.sum()) * (page_bytes(w, t) + (2 * w.P * (w.d // 32) * 4 if outl else 0))
            uni[wl.TIER_NAMES[t] + ("_outliers" if outl else "")] = {
                "attention_avg_us": us, "selected_bytes": b_sel, "achieved_GBps": b_sel / (us * 1e3)}
            for l in ulayers:
                l.release()
            del ulayers
            torch.cuda.empty_cache()
        res["uniform_tier_attention"] = uni
        log(f"[bench] attention with every page in one tier: {uni}")
        tier_demotion(w, res, st)
    if not args.no_basis and tiers is None:
        shared_basis(w, args, res, st)
        lowrank(w, args, res, st)
    if tiers is None:
        # dense line for context: the same attention kernel over every page of
        # every row (k = Np, no score and no selection)
        dsel = torch.arange(w.Np, dtype=torch.int32, device="cuda").repeat(w.B, w.Hkv, 1).contiguous()
        dcnt = torch.full((w.B, w.Hkv), w.Np, dtype=torch.int32, device="cuda")
        dout = torch.empty((w.B, w.Hq, w.d), dtype=torch.float32, device="cuda")
        dlse = torch.empty((w.B, w.Hq), dtype=torch.float32, device="cuda")
        dws = torch.zeros(max(1, kv.attn_workspace_size(layers[0].L, w.B, w.Np) // 4), dtype=torch.float32,
                          device="cuda")
        dense_us = gavg(lambda li, j: kv.sparse_decode_attn(layers[li].L, qs[li][j], layers[li].pages, layers[li].bt,
                                                            layers[li].seq_lens, dsel, dcnt, dout, dlse, dws))
        dense_b = w.rows * w.Np * page_bytes(w, 0)
        res["dense_attention"] = {"avg_launch_us": dense_us, "kv_bytes": dense_b,
                                  "achieved_GBps": dense_b / (dense_us * 1e3),
                                  "note": "every page of every row through kv_sparse_decode_attn; context only, "
                                          "not the path"}
        log(f"[bench] dense attention (k = Np): {dense_us:.1f} us, {dense_b / (dense_us * 1e3):.0f} GB/s")
        del dsel, dws
    sb = append_summary_build(w, args, st)
    if sb is not None:
        res["append_summary_build"] = sb
    # coverage-mode selection (k per row from the mass prefix) on the headline
    # layers' scores: its kernel time and the k it picks, for context
    cov_sel = [torch.empty((w.B, w.Hkv, w.Np), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
    cov_cnt = [torch.empty((w.B, w.Hkv), dtype=torch.int32, device="cuda") for _ in range(n_layers)]
    for li in range(n_layers):
        hz.score(layers[li], qs[li][0], bufs[li])
    cov = {}
    for c in (0.5, 0.95):
        us = gavg(lambda li, j: kv.page_topk_coverage(layers[li].L, bufs[li].head_scores, bufs[li].lse_partial,
                                                      layers[li].seq_lens, w.Np, c, cov_sel[li], cov_cnt[li]))
        kk = cov_cnt[0].cpu().numpy()
        cov[str(c)] = {"avg_launch_us": us, "k_mean": float(kk.mean()), "k_min": int(kk.min()), "k_max": int(kk.max())}
    res["coverage_topk"] = cov
    log(f"[bench] coverage-mode top-k: {cov}")


def tier_demotion(w, res, st):
    """Tier demotion along the cascade on layer 0's scores: budgets at half of
    the workload's mix, so many pages step down in one call."""
    import numpy as np
    import torch
    from quantized_kv_cache_summary_amd import harness as hz
    from quantized_kv_cache_summary_amd import kvsparse as kv
    layers, qs, bufs, stream = st["layers"], st["qs"], st["bufs"], st["stream"]
    clayer = hz.DeviceLayer(w, layer=0, summaries=None, tier_slots="phys")
    hz.score(layers[0], qs[0][0], bufs[0])
    cb = hz.StepBuffers(w, with_S=True)
    cb.head_scores.copy_(bufs[0].head_scores)
    cb.lse_partial.copy_(bufs[0].lse_partial)
    hz.topk(layers[0], cb)
    level_frac = {t: f for f, t in zip(w.tier_fracs, w.tier_order)}
    caps = [int(0.5 * level_frac.get(t, 0.0) * w.Np) for t in (0, 5, 1, 2, 3)]
    moves = torch.empty((w.B, w.Np, 2), dtype=torch.int32, device="cuda")
    mcount = torch.empty((w.B,), dtype=torch.int32, device="cuda")
    e0, e1, e2 = (torch.cuda.Event(enable_timing=True) for _ in range(3))
    # an untimed plan first (it writes only the move list): first-launch costs
    kv.tier_plan(clayer.L, cb.page_S, clayer.seq_lens, clayer.bt, clayer.page_entry, caps, moves, mcount, 1, 1)
    torch.cuda.synchronize()
    e0.record(stream)
    kv.tier_plan(clayer.L, cb.page_S, clayer.seq_lens, clayer.bt, clayer.page_entry, caps, moves, mcount, 1, 1)
    e1.record(stream)
    entry0 = clayer.page_entry.clone()
    torch.cuda.synchronize()
    e1b = torch.cuda.Event(enable_timing=True)
    e1b.record(stream)
    kv.tier_demote(clayer.L, clayer.pages, clayer.page_entry, clayer.bt, moves, mcount)
    e2.record(stream)
    torch.cuda.synchronize()
    mv = moves.cpu().numpy()
    cnt = mcount.cpu().numpy()
    old_t = (entry0.cpu().numpy().view(np.uint32) >> 29)
    moved_b = 0
    for b in range(w.B):
        for phys, nt in mv[b, :cnt[b]]:
            moved_b += page_bytes(w, int(old_t[phys])) * w.Hkv + page_bytes(w, int(nt)) * w.Hkv
    plan_us, demote_us = e0.elapsed_time(e1) * 1e3, e1b.elapsed_time(e2) * 1e3
    res["tier_demotion"] = {
        "caps": caps, "pages_moved": int(cnt.sum()), "plan_us": plan_us, "demote_us": demote_us,
        "demote_bytes": moved_b, "demote_GBps": moved_b / (demote_us * 1e3) if demote_us > 0 else None,
        "note": "one plan (after an untimed one) and one demotion call, eager, on layer 0's scores; "
                "bytes = K+V read in the old tier plus written in the new one"}
    log(f"[bench] tier demotion: {res['tier_demotion']}")
    clayer.release()


def shared_basis(w, args, res, st):
    """The same layers scored from shared-basis summaries (row basis built from
    each layer's keys, then per-page means and variances), same rotation,
    queries, selection rule, attention and timing."""
    import torch
    from quantized_kv_cache_summary_amd import harness as hz
    layers, qs, bufs, fused = st["layers"], st["qs"], st["bufs"], st["fused"]
    n_layers, nq, stream = st["n_layers"], st["nq"], st["stream"]
    t0 = time.time()
    blayers = [l.with_basis_summaries() for l in layers]
    torch.cuda.synchronize()
    log(f"[bench] shared-basis summaries built in {time.time() - t0:.1f}s")
    bsteps = [hz.SplitStep(blayers[i], bufs[i], 1, fused=fused) for i in range(n_layers)]
    for i in range(args.warmup):
        bsteps[i % n_layers](qs[i % n_layers][(i // n_layers) % nq])
    b_ms, _ = timed_region(lambda li, j: bsteps[li](qs[li][j]), n_layers, nq, args.steps, stream)
    bscore_us, _ = graph_avg_us(lambda li, j: hz.score(blayers[li], qs[li][j], bufs[li]), n_layers, nq, args.steps,
                                stream)
    bsum, bselb = basis_algorithmic_bytes(w, bufs[0].sel_count.cpu().numpy())
    log(f"[bench] shared-basis step {b_ms * 1e3:.1f} us, score {bscore_us:.2f} us")
    res["shared_basis"] = {
        "value": 1e3 / b_ms, "unit": "steps/s", "ms_per_step": b_ms, "steps": args.steps,
        "effective_GBps": (bsum + bselb) / (b_ms / 1e3) / 1e9,
        "pct_hbm_peak": 100.0 * (bsum + bselb) / (b_ms / 1e3) / 1e9 / HBM_PEAK_GBS,
        "algorithmic_bytes_per_step": {"summaries": bsum, "selected_kv": bselb},
        "score_kernel": {"avg_launch_us": bscore_us, "achieved_GBps": bsum / (bscore_us * 1e3),
                         "frac": bsum / (bscore_us * 1e3) / HBM_PEAK_GBS},
        "note": "same layers, queries, selection and attention (fused as in the headline step); summaries = "
                "shared row basis + per-page mean and variances (not the headline's per-page directions)",
    }
    del blayers, bsteps


def lowrank(w, args, res, st):
    """The r8 low-rank score (per-key coordinates in a rank-8 row basis) on the
    same layers: the alternative selector, same selection and attention."""
    import torch
    from quantized_kv_cache_summary_amd import harness as hz
    layers, qs, bufs, fused = st["layers"], st["qs"], st["bufs"], st["fused"]
    n_layers, nq, stream = st["n_layers"], st["nq"], st["stream"]
    t0 = time.time()
    rlayers = [l.with_lowrank_summaries() for l in layers]
    torch.cuda.synchronize()
    log(f"[bench] r8 state built in {time.time() - t0:.1f}s")

    def rstep(li, j):
        hz.decode_step(rlayers[li], qs[li][j], bufs[li], fused=fused)

    for i in range(args.warmup):
        rstep(i % n_layers, (i // n_layers) % nq)
    r_ms, _ = timed_region(rstep, n_layers, nq, args.steps, stream)
    rscore_us, _ = graph_avg_us(lambda li, j: hz.score(rlayers[li], qs[li][j], bufs[li]), n_layers, nq, args.steps,
                                stream)
    coord_b = w.rows * w.Np * w.P * 8 * 2 + w.rows * (8 + 1) * w.d * 4
    _, rselb = algorithmic_bytes(w, bufs[0].sel_count.cpu().numpy())
    log(f"[bench] r8 step {r_ms * 1e3:.1f} us, score {rscore_us:.2f} us")
    res["lowrank_r8"] = {
        "value": 1e3 / r_ms, "unit": "steps/s", "ms_per_step": r_ms, "steps": args.steps,
        "algorithmic_bytes_per_step": {"coordinates": coord_b, "selected_kv": rselb},
        "effective_GBps": (coord_b + rselb) / (r_ms / 1e3) / 1e9,
        "score_kernel": {"avg_launch_us": rscore_us, "achieved_GBps": coord_b / (rscore_us * 1e3),
                         "frac": coord_b / (rscore_us * 1e3) / HBM_PEAK_GBS},
        "note": "same layers, queries, selection rule and attention (fused as in the headline step); pages scored "
                "by the exact log-mass of their keys' rank-8 approximations (an alternative selector, not the "
                "headline's)",
    }
    del rlayers


def other_config(name, args):
    """One of the other workloads of the metric's range, measured like the headline."""
    import torch
    from quantized_kv_cache_summary_amd import workloads as wl
    if name == "heavy70b_128k_host_v":
        return heavy_host_v(wl.WORKLOADS["heavy70b_128k"], args)
    if name == "heavy70b_128k_v_in_hbm":
        w = wl.WORKLOADS["heavy70b_128k"].replace(v_host=False, hot_buffer_frac=0.0)
    else:
        w = wl.WORKLOADS[name]
    res, st = measure_step(w, args, extras=False, label=name)
    sb = append_summary_build(w, args, st)
    if sb is not None:
        res["append_summary_build"] = sb
    if name == "heavy70b_128k_v_in_hbm":
        res["note"] = "the 70B-shaped workload with K and V resident in HBM (no host link)"
    release(st)
    torch.cuda.empty_cache()
    return res


def heavy_host_v(w, args):
    """The 70B-shaped workload as stated: K in HBM, V in pinned device-mapped
    host memory with an HBM hot buffer of 10 % of the (page, KV head) units;
    eager steps, first with the buffer left as set up (a seeded random set:
    the reported value), then with LRU admission before every attention.  Its
    bound is the larger of HBM bytes / 8 TB/s and host-link bytes / the link's
    nominal rate."""
    import torch
    from quantized_kv_cache_summary_amd import harness as hz
    steps = max(1, min(args.steps, 10))
    t0 = time.time()
    layer = hz.DeviceLayer(w, summaries="build", hot_mode="cold")
    log(f"[bench] heavy70b_128k_host_v: set-up {time.time() - t0:.1f}s")
    try:
        runs, sel_counts = mem_runs(w, layer, steps, min(args.warmup, 3), max(args.queries, 2))
    finally:
        layer.release()
        torch.cuda.empty_cache()
    static = runs["iid"]["static"]
    summary_b, selected_b = algorithmic_bytes(w, sel_counts)
    cb = combined_bound(summary_b, selected_b, static)
    return {"value": static["value"], "unit": "steps/s", "ms_per_step": static["ms_per_step"], "steps": steps,
            "algorithmic_bytes_per_step": {"summaries": summary_b, "selected_kv": selected_b},
            "combined_bound": cb,
            "host_link": {"bytes_per_step": static["host_bytes_read_by_attention"],
                          "achieved_GBps": static["host_bytes_read_by_attention"] / (static["attention_us"] * 1e3),
                          "link_peak_GBps": HOST_LINK_GBS},
            "hot_buffer": mem_summary(w, runs, summary_b, selected_b),
            "note": "K in HBM, V in pinned device-mapped host memory, HBM hot buffer of 10 % of the (page, KV "
                    "head) units; value: independent queries with the buffer as set up (seeded random set); "
                    "hot_buffer: static against LRU admission before every attention, with independent and "
                    "with drifting queries; eager steps, HIP events; never the headline value"}


def mem_summary(w, runs, summary_b, selected_b):
    """Static buffer against admission, per query kind: step times, hot shares,
    link bytes and each run's combined bound."""
    out = {"buffer_unit": "(physical page, KV head)", "drift_cosine": DRIFT_COS}
    for kind, r in runs.items():
        st, ad = r["static"], r["admission"]
        out[kind] = {"static": st, "admission": ad,
                     "admission_over_static": ad["ms_per_step"] / st["ms_per_step"],
                     "static_bound": combined_bound(summary_b, selected_b, st),
                     "admission_bound": combined_bound(summary_b, selected_b, ad)}
    out["iid"]["queries"] = "independent draws used in turn"
    out["drift"]["queries"] = (f"q_t = c q_(t-1) + sqrt(1 - c^2) xi_t, c = {DRIFT_COS}: consecutive selections "
                               "share most pages, as decode steps do")
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: this path has no multi-GPU mode (asked for --gpus {args.gpus})",
              file=sys.stderr)
        sys.exit(2)
    import torch
    from quantized_kv_cache_summary_amd import workloads as wl

    if args.workload == "heavy70b_128k_v_in_hbm":
        w = wl.WORKLOADS["heavy70b_128k"].replace(v_host=False, hot_buffer_frac=0.0)
    else:
        w = wl.WORKLOADS[args.workload]
    if w.v_host:
        return mem_main(args, w)
    torch.cuda.set_device(0)
    if args.configs == "auto":
        configs = list(OTHER_CONFIGS) if args.workload == HEADLINE else []
    elif args.configs == "none":
        configs = []
    else:
        configs = [c for c in args.configs.split(",") if c]
    res, st = measure_step(w, args, extras=not args.no_extras, label=args.workload)
    if not args.no_extras:
        headline_extras(w, args, res, st)
    release(st)
    cfg = res.pop("config")
    result = {
        "metric": METRIC,
        "value": res["value"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": res["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys/values with planted hot pages and a sink page; no dataset)",
        "config": cfg,
    }
    for k, v in res.items():
        if k not in ("value", "unit", "ms_per_step", "steps"):
            result[k] = v
    if configs:
        result["configs"] = {}
        for name in configs:
            t0 = time.time()
            result["configs"][name] = other_config(name, args)
            log(f"[bench] {name} done in {time.time() - t0:.1f}s")
    tiers = wl.page_tiers(w)
    if not args.no_cpu_baseline and tiers is None:
        log("[bench] oracle baseline on the host ...")
        result["cpu_baseline"] = cpu_baseline(w, args.cpu_seconds)
    print(json.dumps(result), flush=True)


def selected_units(sel, sel_count, bt, seq_lens, P):
    """Hot-buffer unit phys * Hkv + g of every valid selection entry of one
    step (one per (row, page) the attention reads)."""
    import numpy as np
    B, Hkv, k_max = sel.shape
    npg = np.minimum(bt.shape[1], -(-seq_lens.astype(np.int64) // P))
    idx = np.arange(k_max)[None, None, :]
    ok = (idx < np.clip(sel_count, 0, k_max)[:, :, None]) & (sel >= 0) & (sel < npg[:, None, None])
    b = np.broadcast_to(np.arange(B)[:, None, None], sel.shape)
    g = np.broadcast_to(np.arange(Hkv)[None, :, None], sel.shape)
    return bt[b[ok], sel[ok]].astype(np.int64) * Hkv + g[ok]


HOST_LINK_GBS = 64.0   # PCIe 5.0 x16, one direction, nominal


def combined_bound(summary_b, selected_b, run):
    """The step's bound when K or V of cold units crosses the host link: the
    larger of (HBM bytes / 8 TB/s) and (host-link bytes / the link's nominal
    rate).  Host-link bytes are those the attention reads over the link plus
    those admission copies in."""
    host_b = run["host_bytes_read_by_attention"] + run["host_bytes_copied_by_admission"]
    hbm_b = summary_b + selected_b - run["host_bytes_read_by_attention"]
    t = max(hbm_b / (HBM_PEAK_GBS * 1e9), host_b / (HOST_LINK_GBS * 1e9))
    return {"hbm_bytes": hbm_b, "host_bytes": host_b, "bound_ms": t * 1e3,
            "frac": t * 1e3 / run["ms_per_step"]}


DRIFT_COS = 0.95   # cosine of consecutive queries in the step-to-step locality runs


def mem_queries(w, kind, n):
    """Queries of a host-resident run: "iid", a few independent draws used in
    turn, or "drift", a sequence of n with consecutive cosine DRIFT_COS."""
    from quantized_kv_cache_summary_amd import harness as hz
    if kind == "iid":
        return [hz.queries_device(w, 0, j) for j in range(n)]
    return hz.drift_queries_device(w, n, DRIFT_COS)


def mem_runs(w, layer, K, W, nq):
    """Static buffer and LRU admission, with independent queries and then with
    drifting ones (the buffer reset to its seeded contents in between)."""
    import numpy as np
    iid = mem_queries(w, "iid", nq)
    out = {"iid": {}, "drift": {}}
    out["iid"]["static"], sel_counts = mem_run(w, layer, False, K, W, iid)
    out["iid"]["admission"], _ = mem_run(w, layer, True, K, W, iid)
    layer.set_hot_units(np.zeros(0, np.int64))
    drift = mem_queries(w, "drift", W + K + 6)
    out["drift"]["static"], _ = mem_run(w, layer, False, K, W, drift)
    out["drift"]["admission"], _ = mem_run(w, layer, True, K, W, drift)
    for kind in ("iid", "drift"):
        st, ad = out[kind]["static"], out[kind]["admission"]
        log(f"[bench] {w.name} {kind} queries: static {st['ms_per_step'] * 1e3:.0f} us/step "
            f"(hot share {st['hot_share_of_units_called']:.3f}), admission {ad['ms_per_step'] * 1e3:.0f} us/step "
            f"(hot share {ad['hot_share_of_units_called']:.3f}, {ad['units_copied_per_step']:.0f} units copied)")
    return out, sel_counts


def mem_run(w, layer, admit, K, W, qs):
    """Steps over a host-resident pool with the hot buffer as set up (static)
    or with LRU admission of (page, KV head) units before every attention
    (hz.MemStep), step i using qs[i mod len(qs)]; timed, then an untimed pass
    that measures admission and attention per step and the hot share of the
    units the selection calls."""
    import numpy as np
    import torch
    from quantized_kv_cache_summary_amd import harness as hz
    stream = torch.cuda.current_stream()
    nq = len(qs)
    ms = hz.MemStep(layer, admit=admit)
    for i in range(W):
        ms(qs[i % nq])
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for i in range(K):
        ms(qs[(W + i) % nq])
    b.record(stream)
    torch.cuda.synchronize()
    ms_step = a.elapsed_time(b) / K
    # untimed pass: admission and attention per step, hot share of the units
    # called (before this step's admission), units read over the link
    unit_b = w.P * w.d * 2 * (2 if layer.host_k is not None else 1)
    att, adm, hit, n_sel, cold, copies = [], [], [], [], [], []
    for i in range(min(K, 6)):
        bufs = ms.bufs[ms.t & 1]
        q = qs[(W + K + i) % nq]
        hz.score(layer, q, bufs)
        hz.topk(layer, bufs)
        torch.cuda.synchronize()
        reads = selected_units(bufs.sel.cpu().numpy(), bufs.sel_count.cpu().numpy(), layer.bt_np,
                               layer.seq_lens_np, w.P)
        U = np.unique(reads)
        hot_before = layer.v_hot_slot.cpu().numpy()
        hit.append(float((hot_before[U] >= 0).mean()) if U.size else 0.0)
        n_sel.append(int(U.size))
        ms.t += 1
        ea0, ea1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        if admit:
            ea0.record(stream)
            ms.admit_step(bufs)
            ea1.record(stream)
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        hz.attend(layer, q, bufs)
        e1.record(stream)
        torch.cuda.synchronize()
        att.append(e0.elapsed_time(e1) * 1e3)
        hot_after = layer.v_hot_slot.cpu().numpy()
        cold.append(int((hot_after[reads] < 0).sum()))
        if admit:
            adm.append(ea0.elapsed_time(ea1) * 1e3)
            copies.append(int(ms.ws[0].item()))
    sel_counts = ms.bufs[0].sel_count.cpu().numpy()
    return {"ms_per_step": ms_step, "value": 1e3 / ms_step, "unit": "steps/s", "steps": K,
            "attention_us": float(np.median(att)), "admission_us": float(np.median(adm)) if adm else None,
            "units_copied_per_step": float(np.mean(copies)) if copies else 0.0,
            "hot_share_of_units_called": float(np.mean(hit)), "distinct_units_called": float(np.mean(n_sel)),
            "host_bytes_read_by_attention": float(np.mean(cold)) * unit_b,
            "host_bytes_copied_by_admission": (float(np.mean(copies)) if copies else 0.0) * unit_b,
            "hot_slots": int(layer.v_hot.shape[0]), "buffer_unit": "(physical page, KV head)",
            "unit_bytes": unit_b}, sel_counts


def mem_main(args, w):
    """The host-resident workload: V (and with --mem-kv K too) in pinned,
    device-mapped host memory with an HBM hot buffer of a fixed share of the
    (page, KV head) units.  One layer.  Timed: steps with the hot buffer left
    as set up (the headline value: independent queries), steps with LRU
    admission before every attention (kv_hot_admit), both again with drifting
    queries, and static and admission for mem-kv."""
    import numpy as np
    import torch
    from quantized_kv_cache_summary_amd import harness as hz

    torch.cuda.set_device(0)
    stream = torch.cuda.current_stream()
    K, W = args.steps, args.warmup
    nq = max(args.queries, 2)

    t0 = time.time()
    layer = hz.DeviceLayer(w, summaries="build", hot_mode="cold")
    log(f"[bench] {w.name}: set-up {time.time() - t0:.1f}s")
    runs, sel_counts = mem_runs(w, layer, K, W, nq)
    static, admitted = runs["iid"]["static"], runs["iid"]["admission"]
    layer.release()
    memkv = None
    if args.mem_kv:
        t0 = time.time()
        layer = hz.DeviceLayer(w, summaries="build", hot_mode="cold", host_k=True)
        log(f"[bench] {w.name} mem-kv: set-up {time.time() - t0:.1f}s")
        kv_runs, kv_counts = mem_runs(w, layer, K, W, nq)
        sb_k, selb_k = algorithmic_bytes(w, kv_counts)
        memkv = mem_summary(w, kv_runs, sb_k, selb_k)
        layer.release()

    # the same step with V resident in HBM: the bound a hot buffer holding every
    # unit read would approach
    t0 = time.time()
    hl = hz.DeviceLayer(w, summaries="build", host_v=False)
    hb = hz.StepBuffers(w)
    qh = [hz.queries_device(w, 0, j) for j in range(nq)]
    log(f"[bench] {w.name} with V in HBM: set-up {time.time() - t0:.1f}s")
    for i in range(W):
        hz.whole_step(hl, qh[i % nq], hb)
    torch.cuda.synchronize()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for i in range(K):
        hz.whole_step(hl, qh[(W + i) % nq], hb)
    eb.record(stream)
    torch.cuda.synchronize()
    ms_hbm = ea.elapsed_time(eb) / K
    sb_h, selb_h = algorithmic_bytes(w, hb.sel_count.cpu().numpy())
    v_in_hbm = {"ms_per_step": ms_hbm, "value": 1e3 / ms_hbm, "unit": "steps/s", "steps": K,
                "algorithmic_bytes_per_step": {"summaries": sb_h, "selected_kv": selb_h},
                "effective_GBps": (sb_h + selb_h) / (ms_hbm * 1e6),
                "pct_hbm_peak": 100.0 * (sb_h + selb_h) / (ms_hbm * 1e6) / HBM_PEAK_GBS,
                "note": "same workload and step call with K and V resident in HBM (no host link); "
                        "eager launches, HIP events"}
    log(f"[bench] V in HBM: {ms_hbm * 1e3:.1f} us/step, {v_in_hbm['effective_GBps']:.0f} GB/s")
    del hl, hb, qh
    torch.cuda.empty_cache()

    summary_b, selected_b = algorithmic_bytes(w, sel_counts)
    result = {
        "metric": METRIC,
        "value": static["value"],
        "unit": "steps/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": static["ms_per_step"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded N(0,1) keys/values with planted hot pages; no dataset)",
        "config": {"workload": w.name, "batch": w.B, "q_heads": w.Hq, "kv_heads": w.Hkv, "head_dim": w.d,
                   "page_size": w.P, "ctx": w.ctx, "rank": w.rank, "keep": w.keep,
                   "hot_buffer_frac": w.hot_buffer_frac, "timing": "eager, one layer, HIP events",
                   "value_pool": "pinned device-mapped host memory"},
        "algorithmic_bytes_per_step": {"summaries": summary_b, "selected_kv": selected_b},
        "host_link": {
            "note": "V of selected (page, KV head) units not in the hot buffer is read over the host link by "
                    "the attention kernel",
            "bytes_per_step": static["host_bytes_read_by_attention"],
            "achieved_GBps": static["host_bytes_read_by_attention"] / (static["attention_us"] * 1e3),
            "admission_copy_GBps": (admitted["host_bytes_copied_by_admission"] / (admitted["admission_us"] * 1e3)
                                    if admitted["admission_us"] else None),
            "link_peak_GBps": HOST_LINK_GBS,
        },
        "combined_bound": combined_bound(summary_b, selected_b, static),
        "v_in_hbm": v_in_hbm,
        "hot_buffer": mem_summary(w, runs, summary_b, selected_b),
        "mem_kv": memkv,
        "cpu_baseline": None,
    }
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
