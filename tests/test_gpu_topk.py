"""HIP indexer_topk against the oracle's sort-based top-k, bit-exact (C3), on
synthetic score rows: ties, signed zeros, ragged causal lengths, and rows long
enough to need several reduction levels."""
import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from oracle import oracle as O
from synth import gen

from _hip import f32, i32, note

pytestmark = pytest.mark.gpu


def run_topk(scores: np.ndarray, row_len: np.ndarray, max_row_len: int, k: int, ld=None):
    rows = scores.shape[0]
    ld = ld or scores.shape[1]
    s = torch.full((rows, ld), float("nan"), dtype=torch.float32, device="cuda")
    s[:, :scores.shape[1]] = f32(scores)
    out = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
    ws = dsa.alloc_workspace(dsa.IDX_OP_TOPK, rows, max_row_len, k)
    note(f"indexer_topk rows={rows} max_len={max_row_len} k={k} ws={0 if ws is None else ws.numel()}")
    dsa.indexer_topk(s, i32(row_len), max_row_len, k, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


CASES = [
    # rows, n, k, kind
    (4, 2000, 512, "normal"),
    (4, 2000, 512, "ties"),
    (3, 2000, 512, "equal"),
    (3, 3000, 100, "increasing"),
    (3, 3000, 100, "decreasing"),
    (4, 5000, 700, "signed_zero"),
    (4, 22000, 512, "heavy"),
    (8, 22000, 512, "ties"),
    (4, 36864, 1024, "heavy"),
    (2, 36864, 1024, "ties"),
    (2, 131072, 1024, "normal"),
    (2, 131072, 1024, "ties"),
    (1, 200000, 2048, "heavy"),
    # 32,768-element first-level chunks (they save a level here), a partial last chunk
    (2, 600000, 1024, "ties"),
    (2, 100000, 8192, "normal"),
    # k <= 512 on long rows: the later levels use 4096-element chunks (R = 4)
    (2, 131072, 512, "heavy"),
    (3, 60000, 256, "ties"),
    (3, 1000, 1, "normal"),
    (3, 1000, 7, "ties"),
    # k past 1024 on one chunk: the bound from four set maxima per thread holds for
    # k <= 4096 (k = 4097: no bound, every key live, the register passes)
    (3, 36864, 3000, "heavy"),
    (2, 36864, 4096, "ties"),
    (2, 20000, 4097, "normal"),
    # more live keys than the kernel's LDS list holds: the register passes
    (2, 22000, 512, "equal"),
    (2, 36864, 1024, "equal"),
    (2, 30000, 1024, "increasing"),
]


@pytest.mark.parametrize("rows,n,k,kind", CASES)
def test_topk_bit_exact(rows, n, k, kind):
    x = gen.score_rows_for_topk(rows, n, kind=kind, seed=rows * 7 + k)
    rng = np.random.default_rng(n + k)
    lens = np.full(rows, n, np.int64)
    if rows > 1:
        lens[1:] = rng.integers(1, n + 1, size=rows - 1)
    got = run_topk(x, lens, n, k)
    want = O.topk(x, lens, k)
    for r in range(rows):
        assert np.array_equal(got[r], want[r]), (r, int(lens[r]), np.setdiff1d(got[r], want[r])[:5],
                                                 np.setdiff1d(want[r], got[r])[:5])


# Many rows of one chunk each, as chunked prefill makes them, with edge rows
# throughout the batch (and at its end): empty, one key, exactly k, k + 1, every
# score equal (more live keys than the list holds: the register passes) and NaNs.
MANY_ROWS = [(1100, 36864, 1024), (700, 30000, 1024), (600, 22000, 512), (1100, 36864, 64)]


@pytest.mark.parametrize("rows,n,k", MANY_ROWS)
def test_topk_many_rows_bit_exact(rows, n, k):
    x = gen.score_rows_for_topk(rows, n, kind="heavy", seed=rows + n + k)
    rng = np.random.default_rng(rows + k)
    lens = rng.integers(k + 2, n + 1, size=rows).astype(np.int64)
    lens[[3, 300, rows - 1]] = 0
    lens[[5, 301]] = 1
    lens[[7, 302]] = k
    lens[[9, rows - 2]] = k + 1
    lens[[11, 303]] = n
    x[13, :] = 2.5
    x[15, rng.choice(n, 20, replace=False)] = np.nan
    got = run_topk(x, lens, n, k)
    want = O.topk(x, lens, k)
    bad = [r for r in range(rows) if not np.array_equal(got[r], want[r])]
    assert not bad, (len(bad), bad[:10])


def test_topk_edge_lengths():
    k = 512
    lens = np.array([0, 1, k - 1, k, k + 1, 1023, 1024, 1025, 4096, 4097, 32768], np.int64)
    n = int(lens.max())
    x = gen.score_rows_for_topk(len(lens), n, kind="ties", seed=3)
    got = run_topk(x, lens, n, k, ld=n + 5)
    assert np.array_equal(got, O.topk(x, lens, k))


def test_topk_long_rows_1m():
    n, k = 1 << 20, 1024
    x = gen.score_rows_for_topk(2, n, kind="heavy", seed=9)
    lens = np.array([n, n - 12345], np.int64)
    got = run_topk(x, lens, n, k)
    assert np.array_equal(got, O.topk(x, lens, k))


def test_topk_deterministic():
    x = gen.score_rows_for_topk(8, 40000, kind="ties", seed=1)
    lens = np.full(8, 40000)
    a = run_topk(x, lens, 40000, 1024)
    b = run_topk(x, lens, 40000, 1024)
    assert np.array_equal(a, b)


@pytest.mark.parametrize("n,k", [(3000, 512), (36000, 1024), (200000, 1024)])
def test_topk_nan_inf_and_signed_zero_order(n, k):
    """NaNs of both signs and several payloads rank above +inf and tie among
    themselves (torch.topk's order), -0 equals +0, and infinities sit at the ends:
    bit-exact against the oracle, at one reducing level and at several."""
    rng = np.random.default_rng(n)
    rows = 3
    x = (rng.integers(-20, 21, size=(rows, n)).astype(np.float32) * np.float32(0.5))
    nan_bits = np.array([0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF, 0x7FFFFFFF], dtype=np.uint32)
    for r in range(rows):
        m = [k // 4, k + 37, 3][r]                      # fewer NaNs than k, more than k, a few
        at = rng.choice(n, m, replace=False)
        x[r, at] = nan_bits[rng.integers(0, 5, size=m)].view(np.float32)
        x[r, rng.choice(n, 20, replace=False)] = np.float32(np.inf)
        x[r, rng.choice(n, 20, replace=False)] = np.float32(-np.inf)
        x[r, rng.choice(n, 50, replace=False)] = np.float32(-0.0)
    lens = np.array([n, n - 17, n // 2], np.int64)
    got = run_topk(x, lens, n, k)
    want = O.topk(x, lens, k)
    for r in range(rows):
        assert np.array_equal(got[r], want[r]), (r, np.setdiff1d(got[r], want[r])[:5])
