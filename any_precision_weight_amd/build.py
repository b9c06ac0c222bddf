"""Build libapmoe.so (HIP, gfx950) in-tree with hipcc, and libapmoe_safe.so: the
same sources with APMOE_SAFE_WAITS defined, where every counted wait for vector
memory requests drains all of them (slower, never early).  The tests run both and
require identical output bits.

Usage: python -m any_precision_weight_amd.build
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(ROOT, "_build")
LIB = os.path.join(PKG, "libapmoe.so")
SAFE_LIB = os.path.join(PKG, "libapmoe_safe.so")
# a plain HBM read stream for the benchmark's ceiling (not part of the layer)
PROBE_SRC = "hbm_probe.hip"
PROBE_LIB = os.path.join(PKG, "libhbmprobe.so")
SOURCES = ["api.hip", "route.hip", "gemm.hip", "gemm_tile.hip", "elementwise.hip"]
ARCH = "gfx950"

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # packed fp32 instructions stay off: they are never generated into this library
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-I", os.path.join(ROOT, "include"), "-I", CSRC,
]


def _compile(job) -> str:
    src, variant = job
    out_dir = os.path.join(BUILD, variant)
    obj = os.path.join(out_dir, os.path.splitext(src)[0] + ".o")
    extra = ["-DAPMOE_SAFE_WAITS"] if variant == "safe" else []
    cmd = [HIPCC, *FLAGS, *extra, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src} ({variant}):\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, lib):
    tmp = lib + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, lib)


def build(verbose: bool = False, safe: bool = True) -> str:
    variants = ["main", "safe"] if safe else ["main"]
    for v in variants:
        os.makedirs(os.path.join(BUILD, v), exist_ok=True)
    jobs = [(src, v) for v in variants for src in SOURCES] + [(PROBE_SRC, "main")]
    workers = min(len(jobs), int(os.environ.get("MAX_JOBS", "8")))
    with cf.ThreadPoolExecutor(max_workers=workers) as ex:
        objs = list(ex.map(_compile, jobs))
    n = len(SOURCES)
    _link(objs[:n], LIB)
    if safe:
        _link(objs[n:2 * n], SAFE_LIB)
    _link(objs[-1:], PROBE_LIB)
    if verbose:
        print("built", LIB, "and", SAFE_LIB if safe else "(no safe-wait build)")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
