"""HIP sparse attention over selected slots against the oracle (float64).

Tolerance, from the kernel's arithmetic: scores are float32 sums of exact bf16
products (relative error ~512 * 2^-24 of sum |q_d kv_d|, far below the rest); the
probabilities exp(x - m) are float32 and enter the second product rounded to bf16
(relative error <= 2^-9 each), against float32 accumulation.  So each output element
may differ from the exact one by at most
    2^-9 * (sum_j p_j |kv_j[d]|) / (sum_j p_j)
plus float32 terms; the test allows twice that plus 1e-6 * max |kv|, and 2e-5 *
(1 + |lse|) for the log-sum-exp."""
import math

import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from oracle import oracle as O
from synth import gen

from _hip import GpuWorkload, bf16_tensor, note

pytestmark = pytest.mark.gpu


def run(q_bits, kv_bits, slots, scale, k=None, with_ws=True):
    rows, heads = q_bits.shape[:2]
    k = slots.shape[1] if k is None else k
    q = bf16_tensor(q_bits)
    kv = kv_bits if torch.is_tensor(kv_bits) else bf16_tensor(kv_bits)
    sl = torch.from_numpy(np.ascontiguousarray(slots, dtype=np.int64)).cuda()
    out = torch.full((rows, heads, 512), 99.0, dtype=torch.float32, device="cuda")
    lse = torch.full((rows, heads), 99.0, dtype=torch.float32, device="cuda")
    ws = dsa.alloc_attention_workspace(rows, k, heads) if with_ws else None
    note(f"indexer_sparse_attention rows={rows} heads={heads} k={k} slots={kv.shape[0]} "
         f"ws={0 if ws is None else ws.numel()}")
    dsa.indexer_sparse_attention(q, kv, sl, out, k=k, scale=scale, lse=lse, ws=ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def check(out, lse, q_bits, kv64, slots, scale):
    q64 = O.bf16_bits_to_f64(q_bits)
    o, l = O.sparse_attention(q64, kv64, slots, scale)
    rows, heads = q_bits.shape[:2]
    worst = 0.0
    for r in range(rows):
        sel = slots[r][slots[r] >= 0]
        if sel.size == 0:
            assert np.all(out[r] == 0) and np.all(np.isneginf(lse[r])), f"row {r}: empty list"
            continue
        x = kv64[sel]
        s = scale * (q64[r] @ x.T)
        p = np.exp(s - s.max(1, keepdims=True))
        bound = 2.0 ** -9 * (p @ np.abs(x)) / p.sum(1, keepdims=True)       # [H, D]
        tol = 2 * bound + 1e-6 * np.abs(x).max()
        err = np.abs(out[r] - o[r])
        bad = np.argwhere(err > tol)
        assert bad.size == 0, (f"row {r}: {len(bad)} outputs out of tolerance, first {tuple(bad[0])}: "
                               f"gpu={out[r][tuple(bad[0])]!r} oracle={o[r][tuple(bad[0])]!r} "
                               f"tol={tol[tuple(bad[0])]!r}")
        assert np.all(np.abs(lse[r] - l[r]) <= 2e-5 * (1 + np.abs(l[r]))), (r, lse[r][:4], l[r][:4])
        worst = max(worst, float(np.max(err / tol)))
    return worst


CASES = [
    # rows, heads, k, num_slots, pad_frac, q_sd (larger q_sd: peakier softmax)
    (1, 16, 1, 10, 0.0, 1.0),
    (3, 16, 31, 500, 0.1, 1.0),
    (5, 32, 33, 500, 0.0, 1.0),
    (4, 64, 100, 1000, 0.2, 3.0),
    (7, 128, 64, 300, 0.0, 1.0),
    (32, 16, 512, 30000, 0.0, 1.0),
    (32, 64, 512, 30000, 0.0, 4.0),
    (2, 16, 3000, 40000, 0.05, 2.0),       # several splits per row
    (2, 128, 2048, 40000, 0.0, 1.0),
    (1, 64, 5000, 8000, 0.3, 1.0),         # split lists longer than one slot table
    (1, 16, 65536, 70000, 0.1, 1.0),       # the longest list the entry point accepts
    (3, 128, 777, 20000, 0.0, 2.0),        # four 32-head workgroups per row
]


@pytest.mark.parametrize("rows,heads,k,num_slots,pad,q_sd", CASES)
def test_sparse_attention_matches_oracle(rows, heads, k, num_slots, pad, q_sd):
    q_bits, slots = gen.attention_case(rows, heads, k, num_slots, pad_frac=pad, seed=rows + k, q_sd=q_sd)
    kv_bits = gen.kv_states(num_slots, seed=k)
    scale = 1 / math.sqrt(512)
    out, lse = run(q_bits, kv_bits, slots, scale)
    w = check(out, lse, q_bits, O.bf16_bits_to_f64(kv_bits), slots, scale)
    print(f"worst err/tol {w:.3f}, workspace {dsa.attention_workspace_bytes(rows, k, heads)}")


def test_edge_lists():
    # an empty row, a row of padding only, duplicates, k = 0, and the listed slots
    # of a row read through a stride larger than k
    num_slots, heads = 200, 16
    kv_bits = gen.kv_states(num_slots, seed=3)
    q_bits, _ = gen.attention_case(4, heads, 8, num_slots, seed=4)
    slots = np.full((4, 12), 777, np.int64)          # entries past k = 8 must not be read
    slots[0, :8] = -1
    slots[1, :8] = [5, 5, 5, 9, -1, 9, 199, 0]
    slots[2, :8] = [199, -1, -1, -1, -1, -1, -1, 3]
    slots[3, :8] = np.arange(8)
    out, lse = run(q_bits, kv_bits, slots, 0.07, k=8)
    check(out, lse, q_bits, O.bf16_bits_to_f64(kv_bits), slots[:, :8], 0.07)
    out0, lse0 = run(q_bits, kv_bits, slots, 0.07, k=0)
    assert np.all(out0 == 0) and np.all(np.isneginf(lse0))


@pytest.mark.parametrize("k", [40, 3000])
def test_out_of_range_slot_makes_its_row_nan(k):
    num_slots, heads = 5000, 16
    kv_bits = gen.kv_states(num_slots, seed=5)
    q_bits, slots = gen.attention_case(3, heads, k, num_slots, seed=6)
    slots[1, k // 2] = num_slots + 10                  # never read; row 1 becomes NaN
    out, lse = run(q_bits, kv_bits, slots, 1 / math.sqrt(512))
    assert np.all(np.isnan(out[1])) and np.all(np.isnan(lse[1]))
    good = np.array([0, 2])
    check(out[good], lse[good], q_bits[good], O.bf16_bits_to_f64(kv_bits), slots[good], 1 / math.sqrt(512))


def test_attention_over_the_indexer_selections():
    """End to end on the decode-batch shapes: store chain, fused score + top-k with
    physical slots, then attention of 16 query heads over the selected slots of a
    512-dim main KV cache that shares the index cache's block table."""
    wl = gen.config(2, scale=0.1)
    g = GpuWorkload(wl)
    g.store_new()
    out_idx = torch.empty((wl.rows, wl.k), dtype=torch.int32, device="cuda")
    out_slots = torch.empty((wl.rows, wl.k), dtype=torch.int64, device="cuda")
    ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, wl.k)
    note(f"indexer_score_topk {wl.name} rows={wl.rows}")
    dsa.indexer_score_topk(g.q, g.w, g.cache, g.rows, wl.k, out_idx, ws, out_slots=out_slots)
    torch.cuda.synchronize()
    num_slots = wl.num_blocks * wl.block_size
    kv_bits = gen.kv_states(num_slots, seed=11)
    q_bits, _ = gen.attention_case(wl.rows, 16, 1, 1, seed=12)
    slots = out_slots.cpu().numpy()
    # the physical slots are the oracle's translation of the selected positions
    assert np.array_equal(slots, O.translate(out_idx.cpu().numpy(), wl.block_table, wl.row_seq, wl.row_len,
                                             wl.block_size, wl.num_blocks, wl.max_row_len))
    out, lse = run(q_bits, kv_bits, slots, 1 / math.sqrt(512))
    check(out, lse, q_bits, O.bf16_bits_to_f64(kv_bits), slots, 1 / math.sqrt(512))
