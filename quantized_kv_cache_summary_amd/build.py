"""Ahead-of-time build of libkvsparse.so for gfx950 with hipcc.

Every HIP source is compiled with packed-FP32 instructions disabled; the codec
source additionally with floating-point contraction off, because its encoder is
specified operation by operation.  Objects go to ``_build/`` at the repository
root; the shared library lands next to this file.
"""

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OBJ = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libkvsparse.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

SOURCES = {
    "capi.cpp": [],
    "page_score.hip": [],
    "page_topk.hip": [],
    "sparse_attn.hip": [],
    "summary_build.hip": [],
    "basis_build.hip": [],
    "score_basis.hip": [],
    "hot_admit.hip": [],
    "tier_plan.hip": [],
    "score_lowrank.hip": [],
    "codec.hip": ["-ffp-contract=off"],
}

COMMON = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-I", os.path.join(ROOT, "include"),
]


def _compile(name, extra):
    src = os.path.join(CSRC, name)
    obj = os.path.join(OBJ, name + ".o")
    cmd = [HIPCC] + COMMON + extra + ["-c", src, "-o", obj]
    if name.endswith(".cpp"):
        cmd = [HIPCC] + COMMON + extra + ["-x", "hip", "-c", src, "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {name}:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def build(verbose=False):
    os.makedirs(OBJ, exist_ok=True)
    with cf.ThreadPoolExecutor(min(8, len(SOURCES))) as ex:
        objs = list(ex.map(lambda kv: _compile(*kv), SOURCES.items()))
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print("built", LIB)
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
