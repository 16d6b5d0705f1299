"""Key decoding and MFMA operand mapping of the scoring kernels, bit for bit.

The cache is written byte by byte (every e4m3 code, every e2m1 nibble pair, e8m0
block scales over a wide range, arbitrary bf16 patterns), and each query row asks
for one dimension of one key: head h0 holds +1 or -1 at dimension d and zeros
elsewhere, and only h0 carries weight.  The score of key p is then
    max(0, +-value(k_p[d])) * s_p
with a single rounding (the per-key scale), so it must equal the oracle's exact
float64 value rounded once to float32.  Across the 256 rows (128 dimensions, two
signs) and the keys, every code meets every dimension: a wrong code widening
(fp8 -> bf16, e2m1 * 2^e -> bf16), a wrong operand order in either MFMA
(bf16 16x16x32 for bf16 queries, scaled f8f6f4 16x16x128 for fp8 queries, with fp8
or fp4 B) or a wrong scale placement changes some of these scores.
"""
import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from oracle import oracle as O
from synth import gen

from _hip import bf16_tensor, f32, i32, note

pytestmark = pytest.mark.gpu

N_KEYS = 2048
H0 = 37          # the one weighted head (not the first: head order is pinned too)


def key_bytes(kd: str, rng):
    """Logical keys as stored: (per-token code bytes, per-token scale bytes) and the
    float64 keys the oracle decodes from them."""
    n = N_KEYS
    p = np.arange(n)[:, None]
    if kd == "fp8":
        # code of dim d of key p walks all 256 bytes as p varies; NaN codes (0x7F,
        # 0xFF) are replaced by the largest finite value of the same sign
        codes = ((p * 97 + np.arange(128)[None, :] * 37) % 256).astype(np.uint8)
        codes[codes == 0x7F] = 0x7E
        codes[codes == 0xFF] = 0xFE
        scales = (np.exp2(rng.integers(-30, 30, n)) * rng.uniform(1, 2, n)).astype(np.float32)
        keys = O.dequant_fp8(codes, scales)
        return codes, scales.view(np.uint8).reshape(n, 4), keys
    if kd == "fp4":
        nib = ((p * 5 + np.arange(128)[None, :] * 3 + p // 16) % 16).astype(np.uint8)
        e8 = rng.integers(127 - 60, 127 + 60, size=(n, 4)).astype(np.uint8)
        packed = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
        keys = O.dequant_mxfp4(nib, e8)
        return packed, e8, keys
    # bf16: arbitrary finite patterns, over every exponent
    bits = rng.integers(0, 1 << 16, size=(n, 128)).astype(np.uint16)
    exp = (bits >> 7) & 0xFF
    bits[exp == 0xFF] &= np.uint16(0xBFFF)            # no inf / NaN
    bits[exp == 0] &= np.uint16(0x8000)               # no subnormals (signed zeros stay)
    return bits.view(np.uint8).reshape(n, 256), None, O.bf16_bits_to_f64(bits)


def lay_out(kd, codes, scales, bs, table):
    """Cache bytes of the keys behind the block table (the header's layouts)."""
    n = N_KEYS
    tb = {"fp8": 132, "fp4": 68, "bf16": 256}[kd]
    cb = {"fp8": 128, "fp4": 64, "bf16": 256}[kd]
    nblk = table.size
    buf = np.full(nblk * bs * tb, 0xFF, np.uint8)
    for p in range(n):
        b, o = int(table[p // bs]), p % bs
        base = b * bs * tb
        buf[base + o * cb: base + (o + 1) * cb] = codes[p]
        if scales is not None:
            buf[base + bs * cb + o * 4: base + bs * cb + o * 4 + 4] = scales[p]
    return buf


def one_hot_queries():
    """Row 2d + s: head H0 = (+1 if s == 0 else -1) at dimension d; every other
    entry 0; weight 1 on H0 only."""
    rows = 256
    q = np.zeros((rows, 64, 128), np.float32)
    r = np.arange(rows)
    q[r, H0, r // 2] = np.where(r % 2 == 0, 1.0, -1.0)
    w = np.zeros((rows, 64), np.float32)
    w[:, H0] = 1.0
    return q, w


@pytest.mark.parametrize("bs", [64, 32])
@pytest.mark.parametrize("kd,q_fp8", [("fp8", False), ("fp4", False), ("bf16", False),
                                      ("fp8", True), ("fp4", True)])
def test_one_hot_scores_are_exact(kd, q_fp8, bs):
    rng = np.random.default_rng(bs + (7 if q_fp8 else 0) + len(kd))
    codes, scales, keys = key_bytes(kd, rng)
    nblk = N_KEYS // bs
    table = rng.permutation(nblk).astype(np.int32)
    buf = torch.from_numpy(lay_out(kd, codes, scales, bs, table)).cuda()
    dt = {"fp8": dsa.IDX_FP8_E4M3, "fp4": dsa.IDX_MXFP4, "bf16": dsa.IDX_BF16}[kd]
    cache = dsa.kcache(buf, dt, bs, nblk)
    q, w = one_hot_queries()
    rows = q.shape[0]
    bt = i32(table[None, :])
    row_seq = i32(np.zeros(rows))
    row_len = i32(np.full(rows, N_KEYS))
    rd = dsa.rows_desc(bt, row_seq, row_len, N_KEYS)
    out = torch.full((rows, N_KEYS), 7.0, dtype=torch.float32, device="cuda")
    qb = bf16_tensor(gen.f32_to_bf16_bits(q))
    note(f"one-hot scores {kd} keys, {'fp8' if q_fp8 else 'bf16'} queries, bs={bs}")
    if q_fp8:   # e4m3 codes of +-1 (0x38 / 0xB8) and unit query scales
        codes_q = np.where(q > 0, 0x38, np.where(q < 0, 0xB8, 0)).astype(np.uint8)
        qs_host = np.ones((rows, 64), np.float32)
        qc = torch.from_numpy(codes_q).cuda()
        dsa.indexer_score(qc, f32(w), cache, rd, out, q_scale=f32(qs_host))
    else:
        dsa.indexer_score(qb, f32(w), cache, rd, out)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    if q_fp8:   # the oracle decodes the same query codes and scales
        q64 = O.dequant_fp8(codes_q, qs_host)
        assert np.array_equal(q64, q.astype(np.float64))
    else:
        q64 = q.astype(np.float64)
    for r in range(rows):
        # (+ 0: a zero score is +0 whatever sign the float64 sum of zeros took)
        want = O.score(q64[r], w[r].astype(np.float64), keys).astype(np.float32) + np.float32(0)
        g = got[r]
        bad = np.flatnonzero(g.view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, (f"row {r} (dim {r // 2}, sign {'-' if r % 2 else '+'}): {bad.size} keys differ, "
                               f"first p={bad[0]} gpu={g[bad[0]]!r} oracle={want[bad[0]]!r}")
    # every code value met every dimension at least once (the test's own coverage)
    if kd == "fp8":
        assert all(np.unique(codes[:, d]).size == 254 for d in range(128))
    elif kd == "fp4":
        nib = np.empty((N_KEYS, 128), np.uint8)
        nib[:, 0::2], nib[:, 1::2] = codes & 15, codes >> 4
        assert all(np.unique(nib[:, d]).size == 16 for d in range(128))
