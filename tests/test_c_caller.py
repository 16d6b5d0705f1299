"""The C ABI from plain C (tests/c_abi/c_decode_step.c): the header compiles as strict
C11, the caller builds against the library with the host C compiler, and on the GPU
its fp8 store + fused score/top-k selections (three rows, two on one sequence, a
shuffled block table) agree with the oracle's."""
import os
import shutil
import subprocess

import numpy as np
import pytest

import sparse_attention_token_store_amd as dsa
from sparse_attention_token_store_amd import build as B
from oracle import oracle as O

from _hip import note
from _parity import RTOL, check_selection

HEADER = os.path.join(B.ROOT, "include", "dsa_indexer.h")
ROCM = os.environ.get("ROCM_PATH", "/opt/rocm")


def test_header_is_strict_c11(tmp_path):
    cc = shutil.which("gcc") or shutil.which("cc")
    if not cc:
        pytest.skip("no host C compiler")
    src = tmp_path / "h.c"
    src.write_text('#include "dsa_indexer.h"\nint main(void) { return IDX_ABI_VERSION == 2 ? 0 : 1; }\n')
    r = subprocess.run([cc, "-std=c11", "-pedantic", "-Wall", "-Wextra", "-Werror", "-I", os.path.dirname(HEADER),
                        str(src), "-o", str(tmp_path / "h")], capture_output=True, text=True)
    assert r.returncode == 0, r.stderr


@pytest.mark.skipif(not os.path.exists(dsa.LIB_PATH), reason="library not built")
def test_c_caller_builds(tmp_path):
    if not (shutil.which("gcc") or shutil.which("cc")) or not os.path.exists(os.path.join(ROCM, "include", "hip")):
        pytest.skip("no host C compiler or HIP headers")
    out = B.build_c_caller(str(tmp_path / "c_decode_step"))
    assert os.path.exists(out)


def read_result(path):
    raw = open(path, "rb").read()
    off = 0

    def take(dtype, n):
        nonlocal off
        a = np.frombuffer(raw, dtype=dtype, count=n, offset=off)
        off += a.nbytes
        return a

    head = take(np.int32, 9)
    assert head[0] == 0x43414249
    nseq, rows, heads, k, bs, num_blocks, max_blocks, max_row_len = (int(v) for v in head[1:])
    seq_len = take(np.int32, nseq)
    table = take(np.int32, nseq * max_blocks).reshape(nseq, max_blocks)
    row_seq = take(np.int32, rows)
    row_len = take(np.int32, rows)
    keys = take(np.uint16, int(seq_len.sum()) * 128).reshape(-1, 128)
    q = take(np.uint16, rows * heads * 128).reshape(rows, heads, 128)
    w = take(np.float32, rows * heads).reshape(rows, heads)
    idx = take(np.int32, rows * k).reshape(rows, k)
    sc = take(np.float32, rows * k).reshape(rows, k)
    assert off == len(raw)
    return dict(seq_len=seq_len, table=table, row_seq=row_seq, row_len=row_len, keys=keys, q=q, w=w, idx=idx,
                sc=sc, k=k, max_row_len=max_row_len)


@pytest.mark.gpu
def test_c_caller_selections_match_the_oracle(tmp_path):
    exe = B.C_CALLER_OUT
    assert os.path.exists(exe), f"{exe} is not built: run `python -m sparse_attention_token_store_amd.build`"
    out = tmp_path / "result.bin"
    note(f"running the C caller {exe}")
    r = subprocess.run([exe, str(out)], capture_output=True, text=True, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    d = read_result(out)
    # the oracle's keys: each sequence's bf16 keys through its own fp8 quantiser
    starts = np.concatenate([[0], np.cumsum(d["seq_len"])])
    seq_keys = [O.dequant_fp8(*O.quant_fp8(O.bf16_bits_to_f32(d["keys"][starts[b]:starts[b + 1]])))
                for b in range(len(d["seq_len"]))]
    o = O.score_rows(O.bf16_bits_to_f64(d["q"]), d["w"].astype(np.float64), seq_keys, d["row_seq"], d["row_len"],
                     d["max_row_len"])
    print(check_selection(d["idx"], o, d["row_len"], d["k"], RTOL["fp8"]))
    # the selected scores are the oracle's scores of those positions, within the score tolerance
    for r_ in range(d["idx"].shape[0]):
        m = min(d["k"], int(d["row_len"][r_]))
        sel = d["idx"][r_, :m]
        want = o[r_, sel]
        tol = RTOL["fp8"] * np.maximum(np.abs(want), 0.01 * np.max(np.abs(o[r_, :int(d["row_len"][r_])])))
        assert np.all(np.abs(d["sc"][r_, :m] - want) <= tol), r_
        assert np.all(np.isneginf(d["sc"][r_, m:]))
