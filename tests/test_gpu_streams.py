"""Calls on different streams at once: two workloads, each with its own workspace and
outputs, queued on two streams with no synchronisation between them, give the same
results as one after the other on the default stream.  (The library keeps no state
across calls other than indexer_score_topk_static's scratch array, which is not used
here.)"""
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from synth import gen

from _hip import GpuWorkload, note

pytestmark = pytest.mark.gpu


def make(cfg, scale):
    wl = gen.config(cfg, scale=scale)
    g = GpuWorkload(wl)
    g.store_new()
    fp8_q = wl.q_dtype == "fp8"
    if fp8_q:
        g.quantise_q()
    q, qs = g.query(fp8_q)
    ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, wl.k)
    out = torch.empty((wl.rows, wl.k), dtype=torch.int32, device="cuda")
    osc = torch.empty((wl.rows, wl.k), dtype=torch.float32, device="cuda")

    def run(stream=None):
        dsa.indexer_score_topk(q, g.w, g.cache, g.rows, wl.k, out, ws, out_scores=osc, q_scale=qs,
                               stream=stream)
    return g, run, out, osc


def test_two_streams_match_sequential():
    a = make(2, 0.1)      # decode rows, bf16 queries
    b = make(4, 0.03)     # prefill rows, fp8 queries
    note("sequential reference of both workloads")
    refs = []
    for _, run, out, osc in (a, b):
        run()
        torch.cuda.synchronize()
        refs.append((out.clone(), osc.clone()))
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    s1.wait_stream(torch.cuda.current_stream())
    s2.wait_stream(torch.cuda.current_stream())
    for rep in range(4):
        for _, _, out, osc in (a, b):
            out.fill_(-9)
            osc.zero_()
        torch.cuda.synchronize()
        note(f"concurrent round {rep}")
        for _ in range(3):  # several calls queued on each stream, interleaved
            a[1](s1)
            b[1](s2)
        torch.cuda.synchronize()
        for (g, _, out, osc), (ro, rs) in zip((a, b), refs):
            assert torch.equal(out, ro), f"round {rep}: {g.wl.name} selections differ"
            assert torch.equal(osc.view(torch.int32), rs.view(torch.int32)), f"round {rep}: {g.wl.name} scores"
