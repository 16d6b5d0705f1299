"""HIP index-K store and fp8 quantiser against the oracle.

Bit-exact where the result is integer (codes) or a correctly rounded fp32 value
(scales) of the same input; the float64 store chain bounds the float32 one."""
import numpy as np
import pytest
import torch

import sparse_attention_token_store_amd as dsa
from oracle import oracle as O
from synth import gen

from _hip import bf16_tensor, i32, i64, note
from _parity import ambiguous_codes

pytestmark = pytest.mark.gpu


def special_vectors(seed=0):
    """bf16 vectors that stress the quantiser: random scales, zero and tiny rows,
    signed zeros, one dominant element, and every bf16 magnitude <= 448 placed beside
    a 448 (so the scale is exactly 1 and x/s = x)."""
    rng = np.random.default_rng(seed)
    v = [rng.standard_normal((300, 128)) * np.exp(rng.uniform(-20, 20, size=(300, 1)))]
    z = np.zeros((4, 128))
    z[1, 3] = -0.0
    z[2, :] = -0.0
    z[3, 7] = 2.0 ** -120                      # amax below 2^-100: unit scale
    v.append(z)
    d = rng.standard_normal((8, 128)) * 1e-3
    d[np.arange(8), rng.integers(0, 128, 8)] = 1e4
    v.append(d)
    bits = np.concatenate([gen.f32_to_bf16_bits(a.astype(np.float32)) for a in v])
    allbf = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32)
    allbf = allbf[np.isfinite(allbf) & (np.abs(allbf) <= 448)]
    pad = (-allbf.size) % 127
    allbf = np.concatenate([allbf, np.zeros(pad, np.float32)]).reshape(-1, 127)
    ex = np.concatenate([np.full((allbf.shape[0], 1), 448.0, np.float32), allbf], 1)
    return np.concatenate([bits, gen.f32_to_bf16_bits(ex)])


def test_quant_fp8_bit_exact():
    bits = special_vectors()
    x = bf16_tensor(bits)
    codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    note(f"indexer_quant_fp8 n_vec={x.shape[0]}")
    dsa.indexer_quant_fp8(x, codes, scales)
    torch.cuda.synchronize()
    oc, os_ = O.quant_fp8(O.bf16_bits_to_f32(bits))
    gc, gs = codes.cpu().numpy(), scales.cpu().numpy()
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32))
    bad = np.argwhere(gc != oc)
    assert bad.size == 0, (bad[:5], gc[tuple(bad[0])], oc[tuple(bad[0])])


def near_tie_vectors():
    """bf16 vectors whose quotients x / s land within 4 fp32 ulps of an e4m3 rounding
    tie (or on it), found by search: for every bf16 amax in [2^-4, 2^10) and every
    tie M between consecutive e4m3 magnitudes, y = bf16(M * s) with s = fl32(amax/448)
    is kept when fl32(y / s) is that close to M.  Each vector holds amax (so the scale
    is s), the hits for that amax with both signs, and zeros."""
    amax = O.bf16_bits_to_f32(np.arange(0x3D80, 0x4480, dtype=np.uint16))
    s = (amax / np.float32(448)).astype(np.float32)
    mags = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    ties = ((mags[:-1] + mags[1:]) / 2).astype(np.float32)
    ties = np.append(ties, np.float32(464))
    y = O.bf16_bits_to_f32(gen.f32_to_bf16_bits((ties[None, :] * s[:, None]).astype(np.float32)))
    q = (y / s[:, None]).astype(np.float32)
    dist = np.abs(q.view(np.int32).astype(np.int64) - ties.view(np.int32)[None, :].astype(np.int64))
    hit = (dist <= 4) & (y > 0) & (y <= amax[:, None])
    rows = []
    for i in np.flatnonzero(hit.any(axis=1)):
        v = np.zeros(128, np.float32)
        hv = y[i][hit[i]][:63]
        v[0] = amax[i]
        v[1:1 + hv.size] = hv
        v[64:64 + hv.size] = -hv
        rows.append(v)
    return gen.f32_to_bf16_bits(np.stack(rows)), int(hit.sum()), int((dist[hit] == 0).sum())


@pytest.mark.parametrize("entry", ["quant_fp8", "q_prep"])
def test_quantisers_at_e4m3_ties(entry):
    # the quantisers take the codes of y * (1/s) unless that product is near a tie;
    # here every element is near one, and the codes must still be e4m3(RN32(y / s))
    bits, n_hits, n_exact = near_tie_vectors()
    assert n_hits > 1000 and n_exact > 0
    x = bf16_tensor(bits)
    codes = torch.empty(x.shape, dtype=torch.uint8, device="cuda")
    scales = torch.empty(x.shape[0], dtype=torch.float32, device="cuda")
    note(f"{entry} near-tie vectors n_vec={x.shape[0]} hits={n_hits}")
    if entry == "quant_fp8":
        dsa.indexer_quant_fp8(x, codes, scales)
    else:
        dsa.indexer_q_prep(x.view(-1, 1, 128), None, 0, codes=codes.view(-1, 1, 128), scales=scales.view(-1, 1))
    torch.cuda.synchronize()
    oc, os_ = O.quant_fp8(O.bf16_bits_to_f32(bits))
    assert np.array_equal(scales.cpu().numpy().view(np.uint32), os_.view(np.uint32))
    bad = np.argwhere(codes.cpu().numpy() != oc)
    assert bad.size == 0, bad[:5]


def test_quant_fp8_ragged_and_empty():
    rng = np.random.default_rng(1)
    for n in (1, 15, 17, 1000):
        bits = gen.f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
        x = bf16_tensor(bits)
        codes = torch.zeros((n + 1, 128), dtype=torch.uint8, device="cuda")
        scales = torch.full((n + 1,), -7.0, dtype=torch.float32, device="cuda")
        note(f"indexer_quant_fp8 n_vec={n}")
        dsa.indexer_quant_fp8(x, codes[:n], scales[:n])
        torch.cuda.synchronize()
        oc, os_ = O.quant_fp8(O.bf16_bits_to_f32(bits))
        assert np.array_equal(codes[:n].cpu().numpy(), oc)
        assert np.array_equal(scales[:n].cpu().numpy(), os_)
        assert torch.all(codes[n] == 0) and scales[n].item() == -7.0   # nothing written past n
    e = torch.empty((0, 128), dtype=torch.bfloat16, device="cuda")
    dsa.indexer_quant_fp8(e, torch.empty((0, 128), dtype=torch.uint8, device="cuda"),
                          torch.empty(0, dtype=torch.float32, device="cuda"))


def read_fp8_cache(buf: np.ndarray, bs: int, slots: np.ndarray):
    blk, off = slots // bs, slots % bs
    base = blk * bs * 132
    codes = np.stack([buf[b + o * 128: b + o * 128 + 128] for b, o in zip(base, off)])
    scales = np.array([buf[b + bs * 128 + o * 4: b + bs * 128 + o * 4 + 4].view(np.float32)[0]
                       for b, o in zip(base, off)], np.float32)
    return codes, scales


def read_bf16_cache(buf: np.ndarray, bs: int, slots: np.ndarray):
    return np.stack([buf[s * 256:(s + 1) * 256].view(np.uint16) for s in slots])


@pytest.mark.parametrize("bs", [32, 64])
def test_store_flags0_fp8_bit_exact_and_layout(bs):
    bits = special_vectors(seed=2)
    n = bits.shape[0]
    nb = (n + bs - 1) // bs + 3
    rng = np.random.default_rng(3)
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    slots[5] = -1                                          # skipped token
    buf = torch.full((dsa.cache_bytes(dsa.IDX_FP8_E4M3, bs, nb),), 0xA5, dtype=torch.uint8, device="cuda")
    cache = dsa.kcache(buf, dsa.IDX_FP8_E4M3, bs, nb)
    note(f"index_k_store flags=0 fp8 bs={bs} n={n}")
    dsa.index_k_store(bf16_tensor(bits), None, i64(slots), cache, 0)
    torch.cuda.synchronize()
    host = buf.cpu().numpy()
    keep = slots >= 0
    gc, gs = read_fp8_cache(host, bs, slots[keep])
    oc, os_ = O.quant_fp8(O.bf16_bits_to_f32(bits[keep]))
    assert np.array_equal(gc, oc)
    assert np.array_equal(gs.view(np.uint32), os_.view(np.uint32))
    # every byte the store did not own is untouched
    owned = np.zeros(host.size, bool)
    for s in slots[keep]:
        b, o = s // bs, s % bs
        owned[b * bs * 132 + o * 128: b * bs * 132 + o * 128 + 128] = True
        owned[b * bs * 132 + bs * 128 + o * 4: b * bs * 132 + bs * 128 + o * 4 + 4] = True
    assert np.all(host[~owned] == 0xA5)


def test_store_flags0_bf16_copies_bits():
    rng = np.random.default_rng(4)
    bits = gen.f32_to_bf16_bits(rng.standard_normal((200, 128)).astype(np.float32))
    bs, nb = 32, 8
    slots = rng.permutation(nb * bs)[:200].astype(np.int64)
    buf = torch.zeros((dsa.cache_bytes(dsa.IDX_BF16, bs, nb),), dtype=torch.uint8, device="cuda")
    note("index_k_store flags=0 bf16")
    dsa.index_k_store(bf16_tensor(bits), None, i64(slots), dsa.kcache(buf, dsa.IDX_BF16, bs, nb), 0)
    torch.cuda.synchronize()
    assert np.array_equal(read_bf16_cache(buf.cpu().numpy(), bs, slots), bits)


CHAIN_CASES = [
    # flags, rope_base, rope_dim, positions
    (7, 10000.0, 64, "near1m"),
    (7, 160000.0, 64, "mixed"),
    (7, 10000.0, 128, "mixed"),
    (7, 10000.0, 2, "mixed"),
    (1, 10000.0, 64, "mixed"),
    (2, 10000.0, 64, "near1m"),
    (4, 10000.0, 64, "mixed"),
    (6, 10000.0, 32, "mixed"),
]


@pytest.mark.parametrize("flags,base,rope_dim,posk", CHAIN_CASES)
def test_store_chain_fp8(flags, base, rope_dim, posk):
    rng = np.random.default_rng(flags * 131 + rope_dim)
    n, bs, nb = 1000, 64, 20
    bits = gen.f32_to_bf16_bits((rng.standard_normal((n, 128)) * rng.uniform(0.1, 10, (n, 1))).astype(np.float32))
    pos = (1048575 - rng.integers(0, 4096, n)) if posk == "near1m" else rng.integers(0, 1 << 20, n)
    pos = pos.astype(np.int32)
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    buf = torch.zeros((dsa.cache_bytes(dsa.IDX_FP8_E4M3, bs, nb),), dtype=torch.uint8, device="cuda")
    dbg = torch.empty((n, 128), dtype=torch.float32, device="cuda")
    note(f"index_k_store flags={flags} base={base} rope_dim={rope_dim} n={n}")
    dsa.index_k_store(bf16_tensor(bits), i32(pos), i64(slots), dsa.kcache(buf, dsa.IDX_FP8_E4M3, bs, nb),
                      flags, 1e-6, base, rope_dim, prequant_dbg=dbg)
    torch.cuda.synchronize()
    y64 = O.store_chain(bits, pos, flags, 1e-6, base, rope_dim)
    yg = dbg.cpu().numpy().astype(np.float64)
    amax = np.abs(y64).max(axis=1, keepdims=True)
    assert np.all(np.abs(yg - y64) <= 1e-5 * amax), np.max(np.abs(yg - y64) / amax)
    gc, gs = read_fp8_cache(buf.cpu().numpy(), bs, slots)
    # the quantiser on the kernel's own float32 rows: codes and scales bit-exact
    pc, ps = O.quant_fp8(dbg.cpu().numpy())
    bad = np.argwhere(gc != pc)
    assert bad.size == 0, (bad[:5], gc[tuple(bad[0])], pc[tuple(bad[0])])
    assert np.array_equal(gs.view(np.uint32), ps.view(np.uint32))
    # end to end against the float64 chain
    oc, os_ = O.quant_fp8(y64.astype(np.float32))
    assert np.all(np.abs(gs.astype(np.float64) / os_ - 1) <= 1e-5)
    diff = gc != oc
    amb = ambiguous_codes(y64)
    assert not np.any(diff & ~amb), np.argwhere(diff & ~amb)[:5]
    # where they differ the two codes are neighbours (same sign, adjacent magnitude)
    if diff.any():
        a, b = gc[diff].astype(int), oc[diff].astype(int)
        assert np.all((a & 0x80) == (b & 0x80)) and np.all(np.abs((a & 0x7F) - (b & 0x7F)) <= 1)


def test_store_chain_bf16_cache():
    rng = np.random.default_rng(9)
    n, bs, nb = 300, 32, 12
    bits = gen.f32_to_bf16_bits(rng.standard_normal((n, 128)).astype(np.float32))
    pos = rng.integers(0, 1 << 20, n).astype(np.int32)
    slots = rng.permutation(nb * bs)[:n].astype(np.int64)
    buf = torch.zeros((dsa.cache_bytes(dsa.IDX_BF16, bs, nb),), dtype=torch.uint8, device="cuda")
    dbg = torch.empty((n, 128), dtype=torch.float32, device="cuda")
    note("index_k_store flags=7 bf16 cache")
    dsa.index_k_store(bf16_tensor(bits), i32(pos), i64(slots), dsa.kcache(buf, dsa.IDX_BF16, bs, nb),
                      7, 1e-6, 10000.0, 64, prequant_dbg=dbg)
    torch.cuda.synchronize()
    y64 = O.store_chain(bits, pos, 7, 1e-6, 10000.0, 64)
    yg = dbg.cpu().numpy()
    amax = np.abs(y64).max(axis=1, keepdims=True)
    assert np.all(np.abs(yg.astype(np.float64) - y64) <= 1e-5 * amax)
    cached = read_bf16_cache(buf.cpu().numpy(), bs, slots)
    # the cache holds the nearest-even bf16 rounding of the kernel's own float32 rows
    assert np.array_equal(cached, O.bf16_round(yg))
    # and, end to end, one bf16 rounding of a value within 1e-5*amax of the exact one
    got = O.bf16_bits_to_f64(cached)
    assert np.all(np.abs(got - y64) <= np.abs(y64) * 2.0 ** -8 + 1e-5 * amax)


def test_store_zero_tokens_is_noop():
    buf = torch.zeros((dsa.cache_bytes(dsa.IDX_FP8_E4M3, 64, 1),), dtype=torch.uint8, device="cuda")
    note("index_k_store n=0")
    dsa.index_k_store(torch.empty((0, 128), dtype=torch.bfloat16, device="cuda"),
                      torch.empty(0, dtype=torch.int32, device="cuda"),
                      torch.empty(0, dtype=torch.int64, device="cuda"),
                      dsa.kcache(buf, dsa.IDX_FP8_E4M3, 64, 1), dsa.IDX_STORE_ALL)
    torch.cuda.synchronize()
    assert torch.all(buf == 0)


def test_store_encoder_on_a_large_float32_sample():
    # The store converts y / s with the hardware e4m3 conversion after a +-448 clamp.
    # Here 2^17 keys (16.8M quotients y / s) go through the chain: half normalised,
    # rotated and rotary-embedded Gaussian rows, half rotary-embedded rows whose
    # elements spread over 20 binades (so the quotients fill e4m3's subnormal range
    # too).  The cache must hold quant_fp8 of the kernel's own float32 rows, bit for
    # bit: every code is e4m3(RN32(y / s)) rounded to nearest even.
    rng = np.random.default_rng(21)
    n, bs = 1 << 17, 64
    half = n // 2
    a = rng.standard_normal((half, 128)) * rng.uniform(0.1, 10, (half, 1))
    b = rng.standard_normal((half, 128)) * np.exp(rng.uniform(-14, 0, (half, 128)))
    buf = torch.zeros((dsa.cache_bytes(dsa.IDX_FP8_E4M3, bs, n // bs),), dtype=torch.uint8, device="cuda")
    cache = dsa.kcache(buf, dsa.IDX_FP8_E4M3, bs, n // bs)
    dbg = torch.empty((n, 128), dtype=torch.float32, device="cuda")
    slots = np.arange(n, dtype=np.int64)
    for lo, x, flags in ((0, a, 7), (half, b, 2)):
        bits = gen.f32_to_bf16_bits(x.astype(np.float32))
        pos = rng.integers(0, 1 << 20, half).astype(np.int32)
        note(f"index_k_store encoder sample flags={flags} n={half}")
        dsa.index_k_store(bf16_tensor(bits), i32(pos), i64(slots[lo:lo + half]), cache, flags,
                          1e-6, 10000.0, 64, prequant_dbg=dbg[lo:lo + half])
    torch.cuda.synchronize()
    y = dbg.cpu().numpy()
    raw = buf.cpu().numpy().reshape(n // bs, bs * 132)
    gc = raw[:, :bs * 128].reshape(n, 128)
    gs = raw[:, bs * 128:].copy().view(np.float32).reshape(n)
    pc, ps = O.quant_fp8(y)
    assert np.array_equal(gs.view(np.uint32), ps.view(np.uint32))
    bad = np.argwhere(gc != pc)
    assert bad.size == 0, (bad.shape[0], bad[:5], y[tuple(bad[0])] / ps[bad[0][0]])
    q = np.abs(y / ps[:, None])
    assert np.sum((q > 0) & (q < 2.0 ** -6)) > 100_000      # the subnormal range was reached
