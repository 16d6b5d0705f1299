"""HIP logical -> physical translation against the oracle (bit-exact: integer work).

indexer_translate on arbitrary index lists (every -1 case included), and the slots
the fused indexer_score_topk writes beside its selections: equal to the standalone
translation of those selections, to the oracle's, and to the slot the store wrote
each selected key to."""
import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from oracle import oracle as O
from synth import gen

from _hip import GpuWorkload, i32, note

pytestmark = pytest.mark.gpu


def run_translate(idx_np, table_np, row_seq_np, row_len_np, wl, max_row_len=None):
    mrl = wl.max_row_len if max_row_len is None else max_row_len
    table, row_seq, row_len = i32(table_np), i32(row_seq_np), i32(row_len_np)
    rows = dsa.rows_desc(table, row_seq, row_len, mrl)
    cache = dsa.KCache(None, dsa.IDX_FP8_E4M3, wl.block_size, wl.num_blocks)
    idx = i32(idx_np)
    out = torch.full(idx.shape, -7, dtype=torch.int64, device="cuda")
    note(f"indexer_translate rows={idx.shape[0]} k={idx.shape[1]}")
    dsa.indexer_translate(idx, cache, rows, out)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("k", [1, 12, 333, 2048])  # (k % 4 == 0: four entries per thread)
def test_translate_arbitrary_indices(k):
    wl = gen.config(2, scale=0.05)
    rng = np.random.default_rng(k)
    rows = wl.rows
    idx = rng.integers(-3, wl.max_row_len + 70, (rows, k)).astype(np.int32)
    idx[:, ::7] = -1
    edge = [0, wl.row_len[0] - 1, wl.row_len[0]]            # first, last visible, one past
    idx[0, :min(3, k)] = edge[:min(3, k)]
    table = wl.block_table.copy()
    table[1, 0] = -5                                         # block ids outside the pool
    table[2, 1] = wl.num_blocks
    row_seq = wl.row_seq.copy()
    row_seq[3] = table.shape[0]                              # sequence ids outside the table
    row_seq[4] = -1
    got = run_translate(idx, table, row_seq, wl.row_len, wl)
    want = O.translate(idx, table, row_seq, wl.row_len, wl.block_size, wl.num_blocks, wl.max_row_len)
    assert np.array_equal(got, want)
    assert np.all(got[3] == -1) and np.all(got[4] == -1)
    # max_row_len cuts every row
    cut = wl.max_row_len // 3
    got = run_translate(idx, table, row_seq, wl.row_len, wl, max_row_len=cut)
    assert np.array_equal(got, O.translate(idx, table, row_seq, wl.row_len, wl.block_size, wl.num_blocks, cut))


def store_slot_of(wl):
    """slot the store was given for (sequence, position), from the generator's slot
    mapping of every stored key"""
    table = {}
    _, slots = wl.prefix_tokens()
    off = 0
    for b, kb in enumerate(wl.keys_bits):
        table[b] = np.full(int(wl.stored_len[b]) + 1 + int((wl.new_seq == b).sum()), -1, np.int64)
        table[b][:kb.shape[0]] = slots[off:off + kb.shape[0]]
        off += kb.shape[0]
    for s, p, sl in zip(wl.new_seq, wl.new_pos, wl.new_slots()):
        table[int(s)][int(p)] = sl
    return table


# (4, 1.0): all 4096 prefill rows
@pytest.mark.parametrize("cfg,scale", [(2, 0.05), (4, 0.01), (5, 0.02), (1, 1.0), (4, 1.0)])
def test_fused_slots(cfg, scale):
    wl = gen.config(cfg, scale=scale)
    g = GpuWorkload(wl)
    g.store_new()
    fp8_q = wl.q_dtype == "fp8"
    if fp8_q:
        g.quantise_q()
    q, qs = g.query(fp8_q)
    k = wl.k
    ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, k)
    a_idx = torch.empty((wl.rows, k), dtype=torch.int32, device="cuda")
    b_idx = torch.empty_like(a_idx)
    slots = torch.full((wl.rows, k), -7, dtype=torch.int64, device="cuda")
    note(f"indexer_score_topk with slots {wl.name} rows={wl.rows} max_len={wl.max_row_len} k={k}")
    dsa.indexer_score_topk(q, g.w, g.cache, g.rows, k, a_idx, ws, q_scale=qs)
    dsa.indexer_score_topk(q, g.w, g.cache, g.rows, k, b_idx, ws, q_scale=qs, out_slots=slots)
    again = torch.empty_like(slots)
    dsa.indexer_translate(b_idx, g.cache, g.rows, again)
    torch.cuda.synchronize()
    assert torch.equal(a_idx, b_idx)              # the slots change nothing else
    idx, sl = b_idx.cpu().numpy(), slots.cpu().numpy()
    assert np.array_equal(sl, again.cpu().numpy())
    assert np.array_equal(sl, O.translate(idx, wl.block_table, wl.row_seq, wl.row_len, wl.block_size,
                                          wl.num_blocks, wl.max_row_len))
    # each selection's slot is where the store wrote that key
    where = store_slot_of(wl)
    for r in range(wl.rows):
        sel = idx[r] >= 0
        assert np.array_equal(sl[r][sel], where[int(wl.row_seq[r])][idx[r][sel]])
        assert np.all(sl[r][~sel] == -1)
