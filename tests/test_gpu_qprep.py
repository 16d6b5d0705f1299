"""HIP indexer_q_prep (the index query's RoPE + Hadamard + fp8 preparation,
[ATOM-1507] "Where") against the oracle's q_prep, with the store chain's rules:
the kernel's own fp32 rows within 1e-5 of the row's largest magnitude of the fp64
chain, bf16 outputs equal to the rounding of those rows, fp8 codes and scales
bit-exactly the quantiser's on those rows, and end to end only codes at an e4m3
rounding midpoint may move by one step.  Plus the rotation-consistency check on
GPU scores: queries prepared with the key's rotation give the scores of the
unrotated pair."""
import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from oracle import oracle as O
from synth import gen

from _hip import GpuWorkload, bf16_tensor, i32, note
from _parity import RTOL, OracleKeys, ambiguous_codes, check_scores, oracle_scores

pytestmark = pytest.mark.gpu

R, H = dsa.IDX_STORE_ROPE, dsa.IDX_STORE_HADAMARD

CASES = [
    # flags, rope_base, rope_dim, rows, heads
    (R | H, 10000.0, 64, 37, 64),        # the pages' query preparation
    (R, 10000.0, 64, 20, 64),            # "Recommended fix" (A): no rotation on the query
    (H, 10000.0, 64, 9, 16),
    (R | H | dsa.IDX_STORE_RMSNORM, 160000.0, 128, 5, 64),
    (0, 10000.0, 64, 3, 8),
]


def bf16_round_bits(y32: np.ndarray) -> np.ndarray:
    """float32 -> bf16 bits, round to nearest even (finite inputs)."""
    u = y32.view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


@pytest.mark.parametrize("flags,base,rope_dim,rows,heads", CASES)
def test_q_prep_matches_oracle(flags, base, rope_dim, rows, heads):
    rng = np.random.default_rng(flags * 17 + rows)
    x = rng.standard_normal((rows, heads, 128)) * rng.uniform(0.1, 10, (rows, heads, 1))
    bits = gen.f32_to_bf16_bits(x.astype(np.float32))
    pos = rng.integers(0, 1 << 20, rows).astype(np.int32)
    n = rows * heads
    out = torch.empty((rows, heads, 128), dtype=torch.bfloat16, device="cuda")
    codes = torch.empty((rows, heads, 128), dtype=torch.uint8, device="cuda")
    scales = torch.empty((rows, heads), dtype=torch.float32, device="cuda")
    dbg = torch.empty((rows, heads, 128), dtype=torch.float32, device="cuda")
    note(f"indexer_q_prep flags={flags} rows={rows} heads={heads}")
    dsa.indexer_q_prep(bf16_tensor(bits), i32(pos), flags, base, rope_dim, out_bf16=out, codes=codes,
                       scales=scales, prequant_dbg=dbg)
    torch.cuda.synchronize()
    y64 = O.q_prep(bits, pos, flags, base, rope_dim).reshape(n, 128)
    yg = dbg.cpu().numpy().reshape(n, 128)
    amax = np.abs(y64).max(axis=1, keepdims=True)
    assert np.all(np.abs(yg.astype(np.float64) - y64) <= 1e-5 * amax)
    # bf16 output: the rounding of the kernel's own rows
    got_bf16 = out.cpu().view(torch.int16).numpy().view(np.uint16).reshape(n, 128)
    assert np.array_equal(got_bf16, bf16_round_bits(yg))
    # fp8: bit-exact on the kernel's rows; end to end only midpoint codes move, by one step
    gc = codes.cpu().numpy().reshape(n, 128)
    gs = scales.cpu().numpy().reshape(n)
    oc_own, os_own = O.quant_fp8(yg)
    assert np.array_equal(gc, oc_own) and np.array_equal(gs.view(np.uint32), os_own.view(np.uint32))
    oc, os_ = O.quant_fp8(y64.astype(np.float32))
    assert np.all(np.abs(gs.astype(np.float64) / os_ - 1) <= 1e-5)
    diff = gc != oc
    assert not np.any(diff & ~ambiguous_codes(y64))
    if diff.any():
        a, b = gc[diff].astype(int), oc[diff].astype(int)
        assert np.all((a & 0x80) == (b & 0x80)) and np.all(np.abs((a & 0x7F) - (b & 0x7F)) <= 1)


def test_q_prep_outputs_are_independent():
    # each output alone equals the same output of a call that asks for all of them
    rng = np.random.default_rng(5)
    bits = gen.f32_to_bf16_bits(rng.standard_normal((6, 64, 128)).astype(np.float32))
    q, pos = bf16_tensor(bits), i32(rng.integers(0, 5000, 6))
    a = torch.empty((6, 64, 128), dtype=torch.bfloat16, device="cuda")
    b = torch.empty_like(a)
    c1, c2 = torch.empty((6, 64, 128), dtype=torch.uint8, device="cuda"), torch.empty((6, 64, 128), dtype=torch.uint8, device="cuda")
    s1, s2 = torch.empty((6, 64), device="cuda"), torch.empty((6, 64), device="cuda")
    note("indexer_q_prep outputs")
    dsa.indexer_q_prep(q, pos, R | H, out_bf16=a, codes=c1, scales=s1)
    dsa.indexer_q_prep(q, pos, R | H, out_bf16=b)
    dsa.indexer_q_prep(q, pos, R | H, codes=c2, scales=s2)
    torch.cuda.synchronize()
    assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(c1, c2) and torch.equal(s1, s2)


def test_rotated_query_and_key_score_as_the_unrotated_pair():
    # decode rows on bf16 keys: stored with the Hadamard (the store's flag) and
    # queried with a Hadamard-rotated query, the scores are the plain q.k scores
    wl = gen.config(1, scale=1.0)
    g = GpuWorkload(wl, key_dtype="bf16")            # keys stored unrotated (flags = 0)
    x, slots = wl.prefix_tokens()
    buf = torch.full_like(g.buf, 0xFF)
    rot = dsa.kcache(buf, dsa.IDX_BF16, wl.block_size, wl.num_blocks)
    note("store rotated keys, prepare rotated queries")
    dsa.index_k_store(g.prefix_x, None, g.prefix_slots, rot, H)
    qr = torch.empty_like(g.q)
    dsa.indexer_q_prep(g.q, None, H, out_bf16=qr)
    out = torch.empty((wl.rows, wl.max_row_len), dtype=torch.float32, device="cuda")
    dsa.indexer_score(qr, g.w, rot, g.rows, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    # the oracle on the same rotated-and-rounded operands, and on the plain pair
    hq = O.bf16_bits_to_f64(qr.cpu().view(torch.int16).numpy().view(np.uint16))
    hk = O.store_chain(x, np.zeros(x.shape[0], np.int64), H, 1e-6, 10000.0, 64)
    hk = O.bf16_bits_to_f64(bf16_round_bits(hk.astype(np.float32)))
    for r in range(wl.rows):
        n = int(wl.row_len[r])
        o = O.score(hq[r], wl.w[r].astype(np.float64), hk[:n])
        check_scores(got[r:r + 1, :n], o[None], [n], RTOL["bf16"])
    # and the plain, unrotated pair agrees within the bf16 rounding of the operands
    plain = oracle_scores(wl, OracleKeys(wl, "bf16"))
    check_scores(got, plain, wl.row_len, 8 * RTOL["bf16"])


@pytest.mark.parametrize("S", [4500, 22000])
def test_asymmetric_rotation_loses_the_needle_on_gpu(S):
    # the pages' root cause on the GPU path end to end: queries prepared with the
    # Hadamard, a needle of typical key norm aligned with sum_h w_h q_h, scored and
    # selected by the fused score + top-512.  Keys stored with the same rotation keep
    # the needle (rank 1 in the oracle); keys stored without it drop it (oracle rank
    # 3544 at S=4500 and 15418 at S=22000, far outside the top 512).
    k = 512
    wl = gen.make([S], key_dtype="bf16", k=k, seed=0, needle_depth=None)
    keys = O.bf16_bits_to_f64(wl.keys_bits[0])[:S]
    q = O.bf16_bits_to_f64(wl.q_bits[0])
    v = (wl.w[0].astype(np.float64)[:, None] * q).sum(0)
    p = S // 2
    typical = np.median(np.linalg.norm(keys, axis=1))
    wl.keys_bits[0][p] = gen.f32_to_bf16_bits((typical * v / np.linalg.norm(v)).astype(np.float32))
    g = GpuWorkload(wl, key_dtype="bf16")
    qr = torch.empty_like(g.q)
    note(f"asymmetric-rotation needle S={S}")
    dsa.indexer_q_prep(g.q, None, H, out_bf16=qr)

    def selected(flags):
        buf = torch.full_like(g.buf, 0xFF)
        cache = dsa.kcache(buf, dsa.IDX_BF16, wl.block_size, wl.num_blocks)
        dsa.index_k_store(g.prefix_x, None, g.prefix_slots, cache, flags)
        ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, k)
        out = torch.empty((wl.rows, k), dtype=torch.int32, device="cuda")
        dsa.indexer_score_topk(qr, g.w, cache, g.rows, k, out, ws)
        torch.cuda.synchronize()
        return set(out[0].cpu().numpy().tolist())

    assert p in selected(H)
    assert p not in selected(0)
