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
C_CALLER_SRC = os.path.join(ROOT, "tests", "c_abi", "c_decode_step.c")   # plain C caller of the ABI
C_CALLER_OUT = os.path.join(ROOT, "tests", "c_abi", "c_decode_step")

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


def build_c_caller(out: str = C_CALLER_OUT) -> str:
    """Compile the plain C caller of the library (tests/c_abi) with the host C
    compiler.  It includes only include/dsa_indexer.h and the HIP runtime API, and
    finds libdsa_indexer.so next to the package through a relative run path."""
    cc = os.environ.get("CC") or shutil.which("gcc") or shutil.which("cc")
    if not cc:
        raise RuntimeError("no host C compiler (gcc or cc) for the C caller of the library")
    rocm = os.environ.get("ROCM_PATH", "/opt/rocm")
    rel = os.path.relpath(PKG, os.path.dirname(os.path.abspath(out)))
    cmd = [cc, "-std=c11", "-O2", "-Wall", "-Wextra", "-Werror", "-D__HIP_PLATFORM_AMD__",
           "-I", os.path.join(ROOT, "include"), "-I", os.path.join(rocm, "include"), C_CALLER_SRC, "-o", out,
           "-L", PKG, "-ldsa_indexer", "-L", os.path.join(rocm, "lib"), "-lamdhip64",
           "-Wl,-rpath,$ORIGIN/" + rel, "-Wl,-rpath," + os.path.join(rocm, "lib")]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("C caller build failed:\n" + r.stdout + r.stderr)
    return out


def build(verbose: bool = False, extra: list[str] | None = None) -> str:
    """Compile every source and link the indexer library (and the benchmark's
    measurement library), then the plain C caller the tests run; returns the
    indexer library's path."""
    os.makedirs(BUILD_DIR, exist_ok=True)
    srcs = [os.path.join(CSRC, s) for s in SOURCES + BENCH_SOURCES]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(lambda s: _compile(s, extra or []), srcs))
    _link(objs[:len(SOURCES)], OUT)
    _link(objs[len(SOURCES):], BENCH_OUT)
    build_c_caller()
    if verbose:
        print(f"built {OUT}, {BENCH_OUT} and {C_CALLER_OUT}")
    return OUT


if __name__ == "__main__":
    build(verbose=True, extra=sys.argv[1:])
