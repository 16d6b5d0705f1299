"""Seeded random sweep over the shapes the entry points accept, each case against the
oracle: indexer_topk (bit-exact, C3) on random lengths, strides, k and value kinds,
rows long enough for several reduction levels; indexer_sparse_attention (within the
bound of its arithmetic) on random head counts, list lengths, padding and scales; and
the fused indexer_score_topk on random workloads, block sizes and key formats, whose
selection must equal the oracle's top-k of the GPU's own scores."""
import math

import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from oracle import oracle as O
from synth import gen

from _hip import GpuWorkload, bf16_tensor, f32, i32, note
from _parity import RTOL, OracleKeys, check_selection, oracle_scores

pytestmark = pytest.mark.gpu

KINDS = ["normal", "ties", "equal", "increasing", "decreasing", "signed_zero", "heavy"]


@pytest.mark.parametrize("seed", range(4))
def test_random_topk(seed):
    rng = np.random.default_rng(1000 + seed)
    for case in range(25):
        rows = int(rng.integers(1, 6))
        n = int(rng.choice([rng.integers(1, 5000), rng.integers(5000, 40000), rng.integers(40000, 300000),
                            rng.integers(300000, 2500000)]))
        if n > 300000:
            rows = 1
        k = int(rng.choice([1, 7, 100, 256, 512, 1000, 1024, 2048, 4097, 8192]))
        kind = str(rng.choice(KINDS))
        x = gen.score_rows_for_topk(rows, n, kind=kind, seed=int(rng.integers(1 << 30)))
        lens = rng.integers(0, n + 1, size=rows)
        lens[0] = n
        ld = n + int(rng.integers(0, 9))
        s = torch.full((rows, ld), float("nan"), dtype=torch.float32, device="cuda")
        s[:, :n] = f32(x)
        out = torch.full((rows, k), -7, dtype=torch.int32, device="cuda")
        ws = dsa.alloc_workspace(dsa.IDX_OP_TOPK, rows, n, k)
        note(f"seed {seed} case {case}: indexer_topk rows={rows} n={n} ld={ld} k={k} kind={kind}")
        dsa.indexer_topk(s, i32(lens), n, k, out, ws)
        torch.cuda.synchronize()
        got, want = out.cpu().numpy(), O.topk(x, lens, k)
        assert np.array_equal(got, want), (case, rows, n, k, kind, lens)


@pytest.mark.parametrize("seed", range(3))
def test_random_sparse_attention(seed):
    rng = np.random.default_rng(2000 + seed)
    for case in range(20):
        heads = int(rng.choice([16, 32, 64, 128]))
        rows = int(rng.integers(1, 9))
        k = int(rng.choice([1, 5, 33, 100, 512, 777, 2049, 5000]))
        num_slots = int(rng.integers(k, 30000))
        pad = float(rng.choice([0.0, 0.05, 0.5]))
        q_sd = float(rng.choice([0.5, 1.0, 3.0]))
        scale = float(rng.choice([1 / math.sqrt(512), 0.01, 0.1]))
        q_bits, slots = gen.attention_case(rows, heads, k, num_slots, pad_frac=pad,
                                           seed=int(rng.integers(1 << 30)), q_sd=q_sd)
        kv_bits = gen.kv_states(num_slots, seed=int(rng.integers(1 << 30)))
        out = torch.empty((rows, heads, 512), dtype=torch.float32, device="cuda")
        lse = torch.empty((rows, heads), dtype=torch.float32, device="cuda")
        ws = dsa.alloc_attention_workspace(rows, k, heads)
        note(f"seed {seed} case {case}: indexer_sparse_attention rows={rows} heads={heads} k={k} "
             f"slots={num_slots} pad={pad} q_sd={q_sd} scale={scale:.4f}")
        dsa.indexer_sparse_attention(bf16_tensor(q_bits), bf16_tensor(kv_bits), torch.from_numpy(slots).cuda(),
                                     out, k=k, scale=scale, lse=lse, ws=ws)
        torch.cuda.synchronize()
        o, l = out.cpu().numpy(), lse.cpu().numpy()
        q64, kv64 = O.bf16_bits_to_f64(q_bits), O.bf16_bits_to_f64(kv_bits)
        oo, ll = O.sparse_attention(q64, kv64, slots, scale)
        for r in range(rows):
            sel = slots[r][slots[r] >= 0]
            if sel.size == 0:
                assert np.all(o[r] == 0) and np.all(np.isneginf(l[r])), (case, r)
                continue
            x = kv64[sel]
            sc = scale * (q64[r] @ x.T)
            p = np.exp(sc - sc.max(1, keepdims=True))
            # bf16 rounding of the probabilities (2^-9 relative), twice, plus float32 terms
            tol = 2 * 2.0 ** -9 * (p @ np.abs(x)) / p.sum(1, keepdims=True) + 1e-6 * np.abs(x).max()
            assert np.all(np.abs(o[r] - oo[r]) <= tol), (case, r, float(np.max(np.abs(o[r] - oo[r]) / tol)))
            assert np.all(np.abs(l[r] - ll[r]) <= 2e-5 * (1 + np.abs(ll[r]))), (case, r)


@pytest.mark.parametrize("seed", range(2))
def test_random_fused_selection(seed):
    rng = np.random.default_rng(3000 + seed)
    for case in range(8):
        cfg = int(rng.choice([1, 2, 3, 4]))
        scale = float(rng.choice([0.3, 1.0, 3.0])) if cfg == 1 else float(rng.choice([0.01, 0.03, 0.1]))
        bs = int(rng.choice([32, 64]))
        kd = None if cfg == 4 else str(rng.choice(["bf16", "fp8"]))
        wl = gen.config(cfg, scale=scale, block_size=bs, seed=int(rng.integers(1000)), key_dtype=kd)
        kd = wl.key_dtype
        k = int(rng.choice([wl.k, 64, 2048]))
        fp8_q = cfg == 4
        note(f"seed {seed} case {case}: {wl.name} scale={scale} bs={bs} {kd} rows={wl.rows} "
             f"max_len={wl.max_row_len} k={k}")
        g = GpuWorkload(wl, key_dtype=kd)
        g.store_new()
        q64 = None
        if fp8_q:
            g.quantise_q()
            q64 = O.dequant_fp8(*O.quant_fp8(O.bf16_bits_to_f32(wl.q_bits)))
        q, qs = g.query(fp8_q)
        sel = torch.full((wl.rows, k), -7, dtype=torch.int32, device="cuda")
        ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, k)
        dsa.indexer_score_topk(q, g.w, g.cache, g.rows, k, sel, ws, q_scale=qs)
        full = torch.empty((wl.rows, wl.max_row_len), dtype=torch.float32, device="cuda")
        dsa.indexer_score(q, g.w, g.cache, g.rows, full, q_scale=qs)
        torch.cuda.synchronize()
        sel = sel.cpu().numpy()
        ok = OracleKeys(wl, kd)
        check_selection(sel, oracle_scores(wl, ok, q64=q64), wl.row_len, k, RTOL[kd], slack=ok.slack())
        assert np.array_equal(sel, O.topk(full.cpu().numpy(), wl.row_len, k)), case
        del g
        torch.cuda.empty_cache()
