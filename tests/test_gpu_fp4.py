"""MXFP4 index keys (e2m1 + e8m0 per 32 dims) on the GPU against the oracle.

The store's code nibbles and e8m0 bytes are bit-exact with the oracle's quant_mxfp4
of the same input (flags 0), and of the kernel's own pre-quantisation rows after the
store chain; decode scoring of fp4 keys with bf16 queries, and prefill scoring with
fp8 queries on the scaled MFMA (block scales = the e8m0 bytes), match the oracle's
scores on the dequantised keys within the fp32-accumulation tolerance; the fused
selection is valid under the same tolerance."""
import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from oracle import oracle as O
from synth import gen

from _hip import GpuWorkload, bf16_tensor, i32, i64, note
from _parity import RTOL, OracleKeys, check_scores, check_selection, oracle_scores

pytestmark = pytest.mark.gpu


def read_fp4_cache(raw: np.ndarray, bs: int, slots: np.ndarray):
    """(code nibbles [n,128], e8m0 bytes [n,4]) of the tokens at `slots`."""
    blk, off = slots // bs, slots % bs
    base = blk * bs * 68
    cb = raw[(base + off * 64)[:, None] + np.arange(64)[None, :]]
    e8 = raw[(base + bs * 64 + off * 4)[:, None] + np.arange(4)[None, :]]
    codes = np.empty((slots.size, 128), np.uint8)
    codes[:, 0::2] = cb & 15
    codes[:, 1::2] = cb >> 4
    return codes, e8


def special_vectors():
    """Random scales over 40 binades, zero and tiny blocks, block maxima at and just
    below powers of two, and every bf16 magnitude <= 6 (both signs) in blocks led by
    a 6 (scale 2^0, so each element is encoded as given: every e2m1 tie included)."""
    rng = np.random.default_rng(0)
    v = [rng.standard_normal((200, 128)) * np.exp(rng.uniform(-14, 14, size=(200, 1)))]
    z = np.zeros((3, 128))
    z[1, 40] = 3.0                         # three all-zero blocks beside a live one
    z[2, :] = 2.0 ** -130                  # e limited to -127
    v.append(z)
    p2 = rng.standard_normal((8, 128)) * 0.1
    for j in range(4):
        p2[:4, 32 * j] = 2.0 ** (j * 3 - 2)               # block max exactly 2^k
        p2[4:, 32 * j] = 2.0 ** (j * 3 - 2) * (1 - 2 ** -8)  # just below (bf16 neighbour)
    v.append(p2)
    bits = np.concatenate([gen.f32_to_bf16_bits(a.astype(np.float32)) for a in v])
    allbf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    allbf = allbf[np.isfinite(allbf) & (np.abs(allbf) <= 6)]
    pad = (-allbf.size) % 31
    allbf = np.concatenate([allbf, np.zeros(pad, np.float32)]).reshape(-1, 31)
    blocks = np.concatenate([np.full((allbf.shape[0], 1), 6.0, np.float32), allbf], 1)
    pad = (-blocks.shape[0]) % 4
    blocks = np.concatenate([blocks, np.zeros((pad, 32), np.float32)]).reshape(-1, 128)
    return np.concatenate([bits, gen.f32_to_bf16_bits(blocks)])


@pytest.mark.parametrize("bs", [32, 64])
def test_store_fp4_bit_exact(bs):
    bits = special_vectors()
    n = bits.shape[0]
    nb = -(-n // bs) + 3
    slots = np.random.default_rng(bs).permutation(nb * bs)[:n].astype(np.int64)
    buf = torch.full((dsa.cache_bytes(dsa.IDX_MXFP4, bs, nb),), 0xFF, dtype=torch.uint8, device="cuda")
    note(f"index_k_store flags=0 MXFP4 n={n} bs={bs}")
    dsa.index_k_store(bf16_tensor(bits), None, i64(slots), dsa.kcache(buf, dsa.IDX_MXFP4, bs, nb), 0)
    torch.cuda.synchronize()
    gc, ge = read_fp4_cache(buf.cpu().numpy(), bs, slots)
    oc, oe = O.quant_mxfp4(O.bf16_bits_to_f32(bits))
    assert np.array_equal(ge, oe), np.argwhere(ge != oe)[:5]
    bad = np.argwhere(gc != oc)
    assert bad.size == 0, (bad[:5], gc[tuple(bad[0])], oc[tuple(bad[0])])


@pytest.mark.parametrize("flags,posk", [(7, "near1m"), (7, "mixed"), (4, "mixed")])
def test_store_chain_fp4(flags, posk):
    rng = np.random.default_rng(flags + len(posk))
    n, bs, nb = 1000, 64, 20
    bits = gen.f32_to_bf16_bits((rng.standard_normal((n, 128)) * rng.uniform(0.1, 10, (n, 1))).astype(np.float32))
    pos = (1048575 - rng.integers(0, 4096, n)) if posk == "near1m" else rng.integers(0, 1 << 20, n)
    pos = pos.astype(np.int32)
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    buf = torch.zeros((dsa.cache_bytes(dsa.IDX_MXFP4, bs, nb),), dtype=torch.uint8, device="cuda")
    dbg = torch.empty((n, 128), dtype=torch.float32, device="cuda")
    note(f"index_k_store flags={flags} MXFP4 n={n}")
    dsa.index_k_store(bf16_tensor(bits), i32(pos), i64(slots), dsa.kcache(buf, dsa.IDX_MXFP4, bs, nb),
                      flags, 1e-6, 10000.0, 64, prequant_dbg=dbg)
    torch.cuda.synchronize()
    y64 = O.store_chain(bits, pos, flags, 1e-6, 10000.0, 64)
    yg = dbg.cpu().numpy()
    amax = np.abs(y64).max(axis=1, keepdims=True)
    assert np.all(np.abs(yg.astype(np.float64) - y64) <= 1e-5 * amax)
    # bit-exact on the kernel's own rows
    gc, ge = read_fp4_cache(buf.cpu().numpy(), bs, slots)
    oc, oe = O.quant_mxfp4(yg)
    assert np.array_equal(ge, oe) and np.array_equal(gc, oc)


SCORE_CASES = [
    # config, scale, block size
    (1, 1.0, 64),
    (1, 0.37, 32),
    (3, 0.03, 64),
    (3, 0.02, 32),
]


@pytest.mark.parametrize("cfg,scale,bs", SCORE_CASES)
def test_score_fp4_keys(cfg, scale, bs):
    wl = gen.config(cfg, scale=scale, block_size=bs)
    assert wl.new_x_bits.shape[0] == 0     # every key comes from the prefix store
    g = GpuWorkload(wl, key_dtype="fp4")
    out = torch.full((wl.rows, wl.max_row_len + 5), 777.0, dtype=torch.float32, device="cuda")
    note(f"indexer_score MXFP4 {wl.name} rows={wl.rows} max_len={wl.max_row_len} bs={bs}")
    dsa.indexer_score(g.q, g.w, g.cache, g.rows, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[:, wl.max_row_len:] == 777.0)
    o = oracle_scores(wl, OracleKeys(wl, "fp4"))
    print(check_scores(got, o, wl.row_len, RTOL["fp4"]))


def test_score_topk_fp4_keys():
    wl = gen.make([3000, 700, 5000, 64, 1], key_dtype="fp4", k=512, block_size=64, seed=4)
    g = GpuWorkload(wl, key_dtype="fp4")
    ws = dsa.alloc_workspace(dsa.IDX_OP_SCORE_TOPK, wl.rows, wl.max_row_len, wl.k)
    out = torch.empty((wl.rows, wl.k), dtype=torch.int32, device="cuda")
    note(f"indexer_score_topk MXFP4 rows={wl.rows}")
    dsa.indexer_score_topk(g.q, g.w, g.cache, g.rows, wl.k, out, ws)
    torch.cuda.synchronize()
    o = oracle_scores(wl, OracleKeys(wl, "fp4"))
    print(check_selection(out.cpu().numpy(), o, wl.row_len, wl.k, RTOL["fp4"]))


def oracle_fp8_q(wl):
    c, sc = O.quant_fp8(O.bf16_bits_to_f32(wl.q_bits))
    return O.dequant_fp8(c, sc)


@pytest.mark.parametrize("scale,bs", [(0.02, 64), (0.05, 32)])
def test_prefill_fp8_queries_fp4_keys(scale, bs):
    # fp8 queries (oracle-quantised from the same bf16 q) against MXFP4 keys on the
    # scaled MFMA: the e8m0 bytes are the B block scales
    wl = gen.config(4, scale=scale, block_size=bs)
    assert wl.new_x_bits.shape[0] == 0
    g = GpuWorkload(wl, key_dtype="fp4")
    g.quantise_q()
    out = torch.full((wl.rows, wl.max_row_len + 3), 555.0, dtype=torch.float32, device="cuda")
    note(f"indexer_score fp8 q x MXFP4 keys rows={wl.rows} max_len={wl.max_row_len} bs={bs}")
    dsa.indexer_score(g.q_codes, g.w, g.cache, g.rows, out, q_scale=g.q_scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    assert np.all(got[:, wl.max_row_len:] == 555.0)
    o = oracle_scores(wl, OracleKeys(wl, "fp4"), q64=oracle_fp8_q(wl))
    print(check_scores(got, o, wl.row_len, RTOL["fp8"]))


def test_prefill_fp4_rows_of_different_sequences():
    # fp8 queries on the decode layout (every row its own sequence): the per-wave
    # direct path of the prefill kernel, with MXFP4 keys
    wl = gen.config(3, scale=0.01)
    g = GpuWorkload(wl, key_dtype="fp4")
    g.quantise_q()
    out = torch.empty((wl.rows, wl.max_row_len), dtype=torch.float32, device="cuda")
    note(f"indexer_score fp8 q x MXFP4 keys, direct path rows={wl.rows}")
    dsa.indexer_score(g.q_codes, g.w, g.cache, g.rows, out, q_scale=g.q_scale)
    torch.cuda.synchronize()
    o = oracle_scores(wl, OracleKeys(wl, "fp4"), q64=oracle_fp8_q(wl))
    print(check_scores(out.cpu().numpy(), o, wl.row_len, RTOL["fp8"]))


def test_prefill_fp4_bad_block_scores_nan():
    wl = gen.config(4, scale=0.02)
    bt = wl.block_table.copy()
    bt[0, 1] = wl.num_blocks + 3
    g = GpuWorkload(wl, key_dtype="fp4", block_table=bt)
    g.quantise_q()
    out = torch.empty((wl.rows, wl.max_row_len), dtype=torch.float32, device="cuda")
    note("indexer_score fp8 q x MXFP4 keys, bad block id")
    dsa.indexer_score(g.q_codes, g.w, g.cache, g.rows, out, q_scale=g.q_scale)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    bs = wl.block_size
    assert np.all(np.isnan(got[:, bs:2 * bs]))
    assert np.all(np.isfinite(got[:, :bs]))
