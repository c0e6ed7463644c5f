"""Summaries of rocprofv3 runs of bench.py: per-kernel HBM traffic and durations.

Counter readings are scaled by what the same counter reports for a device copy
of known size (bench.py --copy-calibration: 3 x 512 MiB read and written).

  python -m quantized_kv_cache_summary_amd.traffic traffic \
      --fetch FETCH.csv --write WRITE.csv --workload llama8b_32k --command "..."
  python -m quantized_kv_cache_summary_amd.traffic stats --stats STATS.csv --workload ... --command "..."
"""

import argparse
import collections
import csv
import hashlib
import json
import os

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
PROFILES = os.path.join(ROOT, "profiles")
# the sources each kernel family is compiled from: a counter reading stays
# valid while their hash is unchanged
KERNEL_SOURCES = {
    "page_score_kernel": ("page_score.hip", "score_tile.h", "device.h", "launch.h"),
    "page_topk_kernel": ("page_topk.hip", "select.h", "device.h", "launch.h"),
    "sparse_attn_kernel": ("sparse_attn.hip", "attn_split.h", "select.h", "tiers.h", "device.h", "launch.h"),
    "summary_build_kernel": ("summary_build.hip", "device.h", "launch.h"),
}
COPY_BYTES = 3 * (512 << 20)


def kernel_family(name):
    return name.replace("void ", "").replace("kvs::", "").split("<")[0].split("(")[0].strip()


def kernel_sources_hash(name):
    """sha256 over the sources of the kernel's family (None for other kernels)."""
    srcs = KERNEL_SOURCES.get(kernel_family(name))
    if srcs is None:
        return None
    h = hashlib.sha256()
    for f in srcs:
        h.update(open(os.path.join(PKG, "csrc", f), "rb").read())
    return h.hexdigest()


def _per_kernel(path, counter):
    agg = collections.defaultdict(list)
    for r in csv.DictReader(open(path)):
        if r["Counter_Name"] == counter:
            agg[r["Kernel_Name"]].append(float(r["Counter_Value"]))
    return agg


def _short(name):
    return name.split("(")[0].replace("void ", "")


def traffic(args):
    fetch = _per_kernel(args.fetch, "FETCH_SIZE")
    write = _per_kernel(args.write, "WRITE_SIZE")
    copy_f = sum(sum(v) for k, v in fetch.items() if "copyBuffer" in k)
    copy_w = sum(sum(v) for k, v in write.items() if "copyBuffer" in k)
    f_factor = COPY_BYTES / (copy_f * 1024.0)
    w_factor = COPY_BYTES / (copy_w * 1024.0)
    rows = []
    entries = {}
    for k in sorted(fetch, key=lambda k: -sum(fetch[k]) / len(fetch[k])):
        if not k.startswith("void kvs::") and not k.startswith("kvs::"):
            continue
        fk = sum(fetch[k]) / len(fetch[k])
        wk = sum(write.get(k, [0.0])) / max(1, len(write.get(k, [])))
        fb, wb = fk * 1024 * f_factor, wk * 1024 * w_factor
        rows.append((_short(k), len(fetch[k]), fk, wk, fb, wb))
        entries[_short(k)] = {"dispatches": len(fetch[k]), "hbm_read_bytes_per_launch": fb,
                              "hbm_write_bytes_per_launch": wb, "hbm_bytes_per_launch": fb + wb,
                              "sources_sha256": kernel_sources_hash(_short(k))}
    os.makedirs(PROFILES, exist_ok=True)
    md = [f"# HBM traffic per dispatch, {args.workload}", "",
          f"Command (two passes, one counter each): `{args.command}`", "",
          f"Calibration: a device copy of 3 x 512 MiB reads as {copy_f:.1f} KiB FETCH_SIZE and "
          f"{copy_w:.1f} KiB WRITE_SIZE, so readings are scaled by {f_factor:.4f} (fetch) and "
          f"{w_factor:.4f} (write).", "",
          "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | read MB (scaled) | written MB (scaled) |",
          "|---|---|---|---|---|---|"]
    for name, n, fk, wk, fb, wb in rows:
        md.append(f"| {name} | {n} | {fk:.1f} | {wk:.1f} | {fb / 1e6:.2f} | {wb / 1e6:.2f} |")
    open(os.path.join(PROFILES, f"traffic_{args.workload}.md"), "w").write("\n".join(md) + "\n")
    json.dump({"workload": args.workload, "command": args.command, "fetch_factor": f_factor,
               "write_factor": w_factor, "kernels": entries},
              open(os.path.join(PROFILES, f"traffic_{args.workload}.json"), "w"), indent=1)
    print("\n".join(md))


def stats(args):
    rows = list(csv.DictReader(open(args.stats)))
    md = [f"# Kernel durations, {args.workload}", "", f"Command: `{args.command}`", "",
          "| kernel | calls | average us | min us | max us | share % |", "|---|---|---|---|---|---|"]
    for r in rows:
        md.append(f"| {_short(r['Name'])} | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | {float(r['Percentage']):.1f} |")
    os.makedirs(PROFILES, exist_ok=True)
    open(os.path.join(PROFILES, f"kernels_{args.workload}.md"), "w").write("\n".join(md) + "\n")
    print("\n".join(md))


def main():
    ap = argparse.ArgumentParser()
    sub = ap.add_subparsers(dest="cmd", required=True)
    t = sub.add_parser("traffic")
    t.add_argument("--fetch", required=True)
    t.add_argument("--write", required=True)
    t.add_argument("--workload", required=True)
    t.add_argument("--command", required=True)
    s = sub.add_parser("stats")
    s.add_argument("--stats", required=True)
    s.add_argument("--workload", required=True)
    s.add_argument("--command", required=True)
    a = ap.parse_args()
    traffic(a) if a.cmd == "traffic" else stats(a)


if __name__ == "__main__":
    main()
