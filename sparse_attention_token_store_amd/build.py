"""Build the HIP library libdsa_indexer.so in-tree for gfx950.

    python -m sparse_attention_token_store_amd.build

Every HIP source is compiled with hipcc for gfx950 only, with correctly rounded
fp32 division/sqrt (the fp8 quantiser depends on it) and packed-fp32 instruction
selection disabled.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import shutil
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
OUT = os.path.join(PKG, "libdsa_indexer.so")
BENCH_OUT = os.path.join(PKG, "libdsa_bench.so")       # measurement kernels of bench.py
BUILD_DIR = os.path.join(ROOT, "_build")

SOURCES = ["abi.cpp", "store.hip", "score_decode.hip", "score_prefill.hip", "topk.hip", "attention.hip"]
BENCH_SOURCES = ["bench_peaks.hip"]

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-fvisibility=hidden",
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall", "-Wno-unused-function",
]


def hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the indexer library)")


def _compile(src: str, extra: list[str]) -> str:
    obj = os.path.join(BUILD_DIR, os.path.basename(src) + ".o")
    cmd = [hipcc(), *FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-c", src, "-o", obj]
    if src.endswith(".cpp"):
        cmd[1:1] = ["-x", "hip"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    msgs = [ln for ln in (r.stdout + r.stderr).splitlines() if "packed-fp32-ops" not in ln and ln.strip()]
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n" + "\n".join(msgs))
    if msgs:
        sys.stderr.write("\n".join(msgs) + "\n")
    return obj


def _link(objs: list[str], out: str) -> None:
    tmp = out + ".tmp"
    cmd = [hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("link failed:\n" + r.stdout + r.stderr)
    os.replace(tmp, out)


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source and link the indexer library (and the benchmark's
    measurement library); returns the indexer library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES + BENCH_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra or []), srcs))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], BENCH_OUT)
    if verbose:
        print(f"built {OUT} and {BENCH_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
