"""The library's host code (argument checks, level plans, split plans, workspace
sizes) built with AddressSanitizer and UndefinedBehaviorSanitizer and driven by
tests/sanitize/host_abi_harness.cpp: every size query over extreme and random
arguments and a refused call of each kind must run clean.  Only the host side is
instrumented (each sanitizer flag follows -Xarch_host); nothing is launched, so no
GPU is needed."""
import concurrent.futures as cf
import os
import subprocess

import pytest

from sparse_attention_token_store_amd import build as B

HARNESS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "sanitize", "host_abi_harness.cpp")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=undefined", "-Xarch_host", "-fno-omit-frame-pointer"]


def test_host_code_is_clean_under_sanitizers(tmp_path):
    try:
        hipcc = B.hipcc()
    except RuntimeError:
        pytest.skip("hipcc not available")
    flags = ["--offload-arch=gfx950", "-O1", "-g", "-std=c++17", "-fhip-fp32-correctly-rounded-divide-sqrt",
             "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-I", os.path.join(B.ROOT, "include")]

    def compile_one(src):
        obj = str(tmp_path / (os.path.basename(src) + ".o"))
        lang = ["-x", "hip"] if src.endswith(".cpp") else []
        r = subprocess.run([hipcc, *lang, *flags, *HOST_SAN, "-c", src, "-o", obj], capture_output=True, text=True)
        assert r.returncode == 0, r.stderr[-3000:]
        return obj

    srcs = [os.path.join(B.CSRC, s) for s in B.SOURCES] + [HARNESS]
    with cf.ThreadPoolExecutor(max_workers=min(8, len(srcs))) as ex:
        objs = list(ex.map(compile_one, srcs))
    exe = str(tmp_path / "host_abi_harness")
    r = subprocess.run([hipcc, "--offload-arch=gfx950", "-Xarch_host", "-fsanitize=address", "-Xarch_host",
                        "-fsanitize=undefined", *objs, "-o", exe], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-3000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:halt_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert r.returncode == 0, (r.stdout + r.stderr)[-3000:]
    assert "refused calls ok 5/5" in r.stdout
    print(r.stdout.strip())
