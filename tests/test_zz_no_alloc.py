"""indexer_score_topk_static (the library's static per-GPU scratch, no allocation)
against indexer_score_topk with a caller workspace: identical selections, selected
scores and slots, bit for bit, on consecutive calls whose sizes shrink (the second
call reuses the scratch the first one filled)."""
import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from synth import gen

from _hip import GpuWorkload, note

pytestmark = pytest.mark.gpu


def run_both(g: GpuWorkload, fp8_q=False):
    wl = g.wl
    q, qs = g.query(fp8_q)
    outs = []
    for static in (False, True):
        idx = torch.full((wl.rows, wl.k), -7, dtype=torch.int32, device="cuda")
        sc = torch.full((wl.rows, wl.k), 3.0, dtype=torch.float32, device="cuda")
        sl = torch.full((wl.rows, wl.k), -7, dtype=torch.int64, device="cuda")
        note(f"indexer_score_topk{'_static' if static else ''} {wl.name} rows={wl.rows} "
             f"max_len={wl.max_row_len} k={wl.k}")
        if static:
            dsa.indexer_score_topk_static(q, g.w, g.cache, g.rows, wl.k, idx, out_scores=sc, q_scale=qs,
                                          out_slots=sl)
        else:
            ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, wl.k)
            dsa.indexer_score_topk(q, g.w, g.cache, g.rows, wl.k, idx, ws, out_scores=sc, q_scale=qs,
                                   out_slots=sl)
        torch.cuda.synchronize()
        outs.append((idx.cpu().numpy(), sc.cpu().numpy(), sl.cpu().numpy()))
    return outs


def assert_same(a, b):
    assert np.array_equal(a[0], b[0])
    assert np.array_equal(a[1].view(np.uint32), b[1].view(np.uint32))
    assert np.array_equal(a[2], b[2])


def test_static_scratch_matches_workspace_on_shrinking_calls():
    # 1: long rows (the top-k needs candidate lists in the scratch too)
    wl = gen.config(5, scale=0.05)
    need = dsa.workspace_bytes(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, wl.k)
    assert dsa.load_library().indexer_workspace_bytes(dsa.IDX_OP_TOPK, wl.rows, wl.max_row_len, wl.k) > 0
    assert need <= dsa.IDX_STATIC_SCRATCH_BYTES
    g = GpuWorkload(wl)
    g.store_new()
    ref, got = run_both(g)
    assert_same(ref, got)
    del g
    # 2: a smaller decode batch, right after: stale scratch contents must not matter
    wl = gen.config(2, scale=0.05)
    g = GpuWorkload(wl)
    g.store_new()
    ref, got = run_both(g)
    assert_same(ref, got)
    assert np.all(got[0][:, :1] >= 0)
    del g
    # 3: smaller still, fp8 queries on the prefill kernel
    wl = gen.config(4, scale=0.01)
    g = GpuWorkload(wl)
    g.quantise_q()
    ref, got = run_both(g, fp8_q=True)
    assert_same(ref, got)

