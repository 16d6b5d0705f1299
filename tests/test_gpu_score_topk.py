"""HIP indexer_score_topk (the fused decode/prefill selection) against the oracle:
selections (C2), selected scores, the A/B Jaccard (C6), full-size workloads."""
import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from oracle import oracle as O
from synth import gen

from _hip import GpuWorkload, note
from _parity import RTOL, OracleKeys, check_scores, check_selection, oracle_scores

pytestmark = pytest.mark.gpu


def fused(g: GpuWorkload, k=None, fp8_q=False):
    wl = g.wl
    k = k or wl.k
    out = torch.full((wl.rows, k), -7, dtype=torch.int32, device="cuda")
    osc = torch.empty((wl.rows, k), dtype=torch.float32, device="cuda")
    ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, k)
    q, qs = g.query(fp8_q)
    note(f"indexer_score_topk {wl.name} {g.key_dtype} rows={wl.rows} max_len={wl.max_row_len} k={k}")
    dsa.indexer_score_topk(q, g.w, g.cache, g.rows, k, out, ws, out_scores=osc, q_scale=qs)
    torch.cuda.synchronize()
    return out.cpu().numpy(), osc.cpu().numpy()


def scores_dev(g: GpuWorkload, fp8_q=False):
    wl = g.wl
    out = torch.empty((wl.rows, wl.max_row_len), dtype=torch.float32, device="cuda")
    q, qs = g.query(fp8_q)
    note(f"indexer_score {wl.name} rows={wl.rows}")
    dsa.indexer_score(q, g.w, g.cache, g.rows, out, q_scale=qs)
    torch.cuda.synchronize()
    return out


def scores_of(g: GpuWorkload, fp8_q=False):
    return scores_dev(g, fp8_q).cpu().numpy()


def topk_of(g: GpuWorkload, scores, k=None):
    """indexer_topk on device score rows [rows, ld] of the workload's rows."""
    wl = g.wl
    k = k or wl.k
    out = torch.full((wl.rows, k), -7, dtype=torch.int32, device="cuda")
    ws = dsa.alloc_workspace(dsa.IDX_OP_TOPK, wl.rows, wl.max_row_len, k)
    note(f"indexer_topk {wl.name} on its own scores rows={wl.rows} k={k}")
    dsa.indexer_topk(scores, g.row_len, wl.max_row_len, k, out, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy()


def check_topk_on_own_scores(g: GpuWorkload, scores, sel, rows=None):
    """C3: the top-k of the GPU's own float32 score rows, standalone and inside the
    fused call (which scores bit-identically), equals the oracle's sort-based top-k
    of those same rows exactly."""
    wl = g.wl
    rows = np.arange(wl.rows) if rows is None else np.asarray(rows)
    host = scores.cpu().numpy() if torch.is_tensor(scores) else scores
    want = O.topk(host[rows], wl.row_len[rows], wl.k)
    alone = topk_of(g, scores if torch.is_tensor(scores) else torch.from_numpy(host).cuda())
    for i, r in enumerate(rows):
        assert np.array_equal(alone[r], want[i]), (f"row {r}: indexer_topk differs from the oracle's top-k "
                                                   f"of the same rows: {np.setdiff1d(alone[r], want[i])[:5]}")
        assert np.array_equal(sel[r], want[i]), f"row {r}: fused selection differs from the oracle's top-k"


CASES = [
    (1, 1.0, "bf16", 64, None),
    (1, 1.0, "bf16", 64, 4000),       # k >= row_len: every position
    (2, 0.1, "fp8", 64, None),
    (2, 0.1, "fp8", 32, 1024),
    (3, 0.03, "fp8", 64, None),
    (5, 0.004, "fp8", 64, None),
]


@pytest.mark.parametrize("cfg,scale,kd,bs,k", CASES)
def test_fused_selection_matches_oracle(cfg, scale, kd, bs, k):
    wl = gen.config(cfg, scale=scale, block_size=bs, key_dtype=kd)
    g = GpuWorkload(wl, key_dtype=kd)
    g.store_new()
    k = k or wl.k
    sel, sc = fused(g, k)
    ok = OracleKeys(wl, kd)
    o = oracle_scores(wl, ok)
    print(check_selection(sel, o, wl.row_len, k, RTOL[kd], slack=ok.slack()))
    # the selected scores are the ones indexer_score produces, bit for bit
    full = scores_of(g)
    for r in range(wl.rows):
        m = min(k, int(wl.row_len[r]))
        assert np.array_equal(sc[r, :m].view(np.uint32), full[r, sel[r, :m]].view(np.uint32))
        assert np.all(np.isneginf(sc[r, m:]))
    if wl.needle_pos[0] >= 0:
        for r in range(wl.rows):
            assert wl.needle_pos[wl.row_seq[r]] in set(sel[r].tolist())


def test_decode_b32_full_size():
    """The benchmark workload at full size: store chain + fused score/top-k."""
    wl = gen.config(2)
    g = GpuWorkload(wl)
    g.store_new()
    sel, _ = fused(g)
    ok = OracleKeys(wl)
    o = oracle_scores(wl, ok)
    st = check_selection(sel, o, wl.row_len, wl.k, RTOL["fp8"], slack=ok.slack())
    print(st)
    sd = scores_dev(g)
    check_scores(sd.cpu().numpy(), o, wl.row_len, RTOL["fp8"], slack=ok.slack())
    check_topk_on_own_scores(g, sd, sel)
    for r in range(wl.rows):
        assert wl.needle_pos[r] in set(sel[r].tolist())


@pytest.mark.parametrize("scale", [0.125, 1.0])
def test_ab_jaccard_bf16_vs_fp8(scale):
    """Same keys stored as bf16 and as fp8: both selections match the oracle, and the
    Jaccard overlap measured on the GPU agrees with the oracle's up to the ambiguous
    positions of the two selections."""
    wl = gen.config(3, scale=scale)
    res = {}
    for kd in ("bf16", "fp8"):
        g = GpuWorkload(wl, key_dtype=kd)
        sel, _ = fused(g)
        ok = OracleKeys(wl, kd)
        o = oracle_scores(wl, ok)
        st = check_selection(sel, o, wl.row_len, wl.k, RTOL[kd])
        res[kd] = (sel, O.topk(o, wl.row_len, wl.k), st)
        del g, o
        torch.cuda.empty_cache()
    amb = res["bf16"][2]["ambiguous"] + res["fp8"][2]["ambiguous"]
    jg = [O.jaccard(res["bf16"][0][r], res["fp8"][0][r])[0] for r in range(wl.rows)]
    jo = [O.jaccard(res["bf16"][1][r], res["fp8"][1][r])[0] for r in range(wl.rows)]
    print("jaccard gpu", np.round(jg, 4), "oracle", np.round(jo, 4), "ambiguous", amb)
    for a, b in zip(jg, jo):
        assert abs(a - b) <= (amb + 1) / wl.k
    for kd in ("bf16", "fp8"):
        for r in range(wl.rows):
            assert wl.needle_pos[r] in set(res[kd][0][r].tolist())


def test_long_decode_b4_full_size():
    """4 x 1,048,576 fp8 keys: 4096 tokens through the store chain, then the fused
    selection over every key."""
    wl = gen.config(5)
    g = GpuWorkload(wl)
    g.store_new()
    sel, _ = fused(g)
    check_topk_on_own_scores(g, scores_dev(g), sel)
    ok = OracleKeys(wl)
    o = oracle_scores(wl, ok)
    print(check_selection(sel, o, wl.row_len, wl.k, RTOL["fp8"], slack=ok.slack()))


@pytest.mark.parametrize("scale", [0.05, 1.0])
def test_prefill_fused_selection(scale):
    """Chunked prefill: fp8 queries, 4096 (or fewer) causal rows on a 32K prefix."""
    wl = gen.config(4, scale=scale)
    g = GpuWorkload(wl)
    g.quantise_q()
    sel, sc = fused(g, fp8_q=True)
    c, s = O.quant_fp8(O.bf16_bits_to_f32(wl.q_bits))
    q64 = O.dequant_fp8(c, s)
    # the oracle scores a sample of rows (every row at small scale)
    rows = np.arange(wl.rows) if wl.rows <= 256 else np.linspace(0, wl.rows - 1, 48).astype(int)
    o = oracle_scores(wl, OracleKeys(wl), rows=rows, q64=q64[rows])
    print(check_selection(sel[rows], o, wl.row_len[rows], wl.k, RTOL["fp8"]))
    # C3 on the GPU's own scores of the same rows (every row's top-k runs on the GPU)
    sd = scores_dev(g, fp8_q=True)
    check_topk_on_own_scores(g, sd, sel, rows=rows if wl.rows <= 256 else np.linspace(0, wl.rows - 1, 256).astype(int))
