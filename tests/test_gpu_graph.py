"""One indexer step captured in a HIP graph: the store of the step's new tokens, the
query quantisation (fp8-query workloads) and the fused score + top-k.  Every
replay, with eager work of the library and of torch between the replays, must give
the eager step's selections and selected scores bit for bit.  (None of the entry
points records a memset or a copy, so nothing but kernels enters the graph.)"""
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from synth import gen

from _hip import GpuWorkload, note

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("cfg,scale", [(2, 0.05), (4, 0.01), (5, 0.004)])
def test_captured_step_replays_match_eager(cfg, scale):
    wl = gen.config(cfg, scale=scale)
    g = GpuWorkload(wl)
    fp8_q = wl.q_dtype == "fp8"
    if fp8_q:
        g.quantise_q()
    q, qs = g.query(fp8_q)
    k = wl.k
    ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, k)
    out = torch.full((wl.rows, k), -7, dtype=torch.int32, device="cuda")
    osc = torch.empty((wl.rows, k), dtype=torch.float32, device="cuda")

    def step(o_idx, o_sc, w_s):
        if wl.new_x_bits.shape[0]:
            dsa.index_k_store(g.new_x, g.new_pos, g.new_slots, g.cache, dsa.IDX_STORE_ALL,
                              wl.rms_eps, wl.rope_base, wl.rope_dim)
        if fp8_q:
            dsa.indexer_quant_fp8(g.q, g.q_codes, g.q_scale)
        dsa.indexer_score_topk(q, g.w, g.cache, g.rows, k, o_idx, w_s, out_scores=o_sc, q_scale=qs)

    note(f"eager step {wl.name} rows={wl.rows} max_len={wl.max_row_len} k={k}")
    step(out, osc, ws)
    torch.cuda.synchronize()
    ref_idx, ref_sc = out.clone(), osc.clone()

    note(f"capture step {wl.name}")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step(out, osc, ws)  # warm-up on the capture stream
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step(out, osc, ws)
    torch.cuda.synchronize()

    other_idx, other_sc = torch.empty_like(out), torch.empty_like(osc)
    other_ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, k)
    for rep in range(3):
        out.fill_(-9)
        osc.zero_()
        torch.cuda.synchronize()
        note(f"replay {rep} {wl.name}")
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out, ref_idx), f"replay {rep}: selections differ"
        assert torch.equal(osc.view(torch.int32), ref_sc.view(torch.int32)), f"replay {rep}: scores differ"
        # eager work between replays: the same step into other buffers, and torch ops
        step(other_idx, other_sc, other_ws)
        _ = torch.randn(1 << 20, device="cuda").sum().item()
        torch.cuda.synchronize()
        assert torch.equal(other_idx, ref_idx)


def test_captured_decode_step_with_slots_and_attention():
    """A decode step through to the attention: the store of the new tokens, the fused
    selection with physical slots, and the sparse attention (split and merge kernels)
    over those slots, captured once and replayed with eager work in between; every
    replay must equal the eager step bit for bit."""
    wl = gen.config(2, scale=0.05)
    g = GpuWorkload(wl)
    k, heads = wl.k, 16
    num_slots = wl.num_blocks * wl.block_size
    gen_ = torch.Generator(device="cuda")
    gen_.manual_seed(11)
    kv = torch.randn((num_slots, dsa.KV_DIM), device="cuda", generator=gen_).to(torch.bfloat16)
    qa = torch.randn((wl.rows, heads, dsa.KV_DIM), device="cuda", generator=gen_).to(torch.bfloat16)
    ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, k)
    aws = dsa.alloc_attention_workspace(wl.rows, k, heads)
    idx = torch.empty((wl.rows, k), dtype=torch.int32, device="cuda")
    slots = torch.empty((wl.rows, k), dtype=torch.int64, device="cuda")
    out = torch.empty((wl.rows, heads, dsa.KV_DIM), dtype=torch.float32, device="cuda")
    lse = torch.empty((wl.rows, heads), dtype=torch.float32, device="cuda")

    def step():
        dsa.index_k_store(g.new_x, g.new_pos, g.new_slots, g.cache, dsa.IDX_STORE_ALL,
                          wl.rms_eps, wl.rope_base, wl.rope_dim)
        dsa.indexer_score_topk(g.q, g.w, g.cache, g.rows, k, idx, ws, out_slots=slots)
        dsa.indexer_sparse_attention(qa, kv, slots, out, lse=lse, ws=aws)

    note(f"eager decode step with attention rows={wl.rows} k={k} heads={heads} ws={aws.numel()}")
    step()
    torch.cuda.synchronize()
    ref = [t.clone() for t in (idx, slots, out, lse)]
    assert bool((ref[1] >= 0).any())  # (rows shorter than k pad with -1)

    note("capture decode step with attention")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        step()
        side.synchronize()
        with torch.cuda.graph(graph, stream=side):
            step()
    torch.cuda.synchronize()
    for rep in range(3):
        for t in (idx, slots, out, lse):
            t.zero_()
        torch.cuda.synchronize()
        note(f"replay {rep} decode step with attention")
        graph.replay()
        torch.cuda.synchronize()
        for name, t, r in zip(("idx", "slots", "out", "lse"), (idx, slots, out, lse), ref):
            assert torch.equal(t.view(torch.uint8), r.view(torch.uint8)), f"replay {rep}: {name} differs"
        # eager work between replays: the library's own step and a torch reduction
        step()
        _ = torch.randn(1 << 20, device="cuda").sum().item()
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), ref[2].view(torch.uint8))
