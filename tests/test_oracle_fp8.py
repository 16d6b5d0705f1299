"""Pins of the oracle's fp8 e4m3 codec and per-vector quantiser against things other
than itself: values fixed by the OCP e4m3fn format definition, torch's independent
float8_e4m3fn conversion, exact rational rounding, and hand-worked examples."""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O


def f32(v):
    return np.asarray(v, dtype=np.float32)


def test_decode_format_definition_values():
    # e4m3fn: bias 7, 3 mantissa bits, no infinities, NaN only at S.1111.111
    d = O.e4m3_decode(np.array([0x00, 0x01, 0x07, 0x08, 0x38, 0x7E, 0x80, 0xB8, 0xFE, 0x7F, 0xFF], np.uint8))
    assert d[0] == 0.0 and not math.copysign(1, d[0]) < 0
    assert d[1] == 2.0 ** -9                    # smallest subnormal: 2^-6 * 1/8
    assert d[2] == 7 * 2.0 ** -9                # largest subnormal
    assert d[3] == 2.0 ** -6                    # smallest normal
    assert d[4] == 1.0                          # e=7, m=0
    assert d[5] == 448.0                        # e=15, m=6: 2^8 * 1.75
    assert d[6] == 0.0 and math.copysign(1, d[6]) < 0
    assert d[7] == -1.0
    assert d[8] == -448.0
    assert np.isnan(d[9]) and np.isnan(d[10])


def test_decode_table_strictly_increasing():
    t = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    assert np.all(np.diff(t) > 0)
    assert t.size == 127


def test_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert codes.size == 254
    vals = O.e4m3_decode(codes)
    back = O.e4m3_encode(f32(vals))
    assert np.array_equal(back, codes)          # includes -0 -> 0x80


def _torch_e4m3(x32):
    return torch.from_numpy(np.ascontiguousarray(x32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def _pin_sample():
    """fp32 values that stress rounding: every midpoint between adjacent codes and
    its float32 neighbours, all bf16 values up to 464, and random fp32 in range."""
    t = O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = f32((t[:-1] + t[1:]) / 2)
    up = np.nextafter(mids, np.float32(np.inf))
    dn = np.nextafter(mids, np.float32(-np.inf))
    bf = (np.arange(0, 1 << 16, dtype=np.uint32) << 16).view(np.float32)
    bf = bf[np.isfinite(bf)]
    rng = np.random.default_rng(7)
    e = rng.uniform(-14, math.log2(464), size=1 << 20)
    rnd = f32(np.exp2(e) * rng.choice([-1, 1], size=e.size))
    x = np.concatenate([mids, up, dn, f32(t), bf, rnd, -mids, -up, -dn])
    return x[np.abs(x) <= 464].astype(np.float32)


def test_encode_matches_torch_float8_e4m3fn():
    # torch rounds to nearest even and saturates to 448 for |x| <= 464 (it returns
    # NaN above, where ours saturates, so the comparison stays within 464).
    x = _pin_sample()
    ours = O.e4m3_encode(x)
    ref = _torch_e4m3(x)
    bad = np.nonzero(ours != ref)[0]
    assert bad.size == 0, (x[bad[:10]], ours[bad[:10]], ref[bad[:10]])


def test_encode_exact_rational_bruteforce():
    table = [Fraction(float(v)) for v in O.e4m3_decode(np.arange(0x7F, dtype=np.uint8))]
    rng = np.random.default_rng(11)
    xs = f32(np.exp2(rng.uniform(-13, 9.2, size=3000)) * rng.choice([-1, 1], size=3000))
    got = O.e4m3_encode(xs)
    for x, g in zip(xs.tolist(), got.tolist()):
        a = abs(Fraction(x))
        if a >= 448:
            want = 126
        else:
            dist = [abs(a - v) for v in table]
            best = min(dist)
            cands = [c for c, dd in enumerate(dist) if dd == best]
            want = cands[0] if len(cands) == 1 else [c for c in cands if c % 2 == 0][0]
        if math.copysign(1.0, x) < 0:
            want |= 0x80
        assert g == want, (x, g, want)


def test_encode_saturates_and_keeps_sign():
    x = f32([448.0, 460.0, 464.0, 465.0, 1e30, -500.0, -0.0, -1e-30, 2.0 ** -10, -(2.0 ** -10)])
    got = O.e4m3_encode(x).tolist()
    # 464 is the midpoint of 448 and the (non-finite) next step: ties-to-even -> 448
    assert got == [0x7E, 0x7E, 0x7E, 0x7E, 0x7E, 0xFE, 0x80, 0x80, 0x00, 0x80]


def test_quant_hand_worked_example():
    # amax = 3.5 -> s = 3.5/448 = 2^-7 exactly, so x/s = 128 x exactly:
    #   1 -> 128 = 2^7  -> e=14,m=0 -> 0x70       -2 -> -256 = -2^8 -> 0xF8
    #   0.5 -> 64 = 2^6 -> e=13 -> 0x68           3.5 -> 448 -> 0x7E
    #   0 -> 0x00, -0 -> 0x80
    #   0.01171875 = 3*2^-8 -> 1.5 = 2^0*1.5 -> e=7,m=4 -> 0x3C
    #   2^-16 -> 2^-9 = smallest subnormal -> 0x01
    #   3*2^-18 -> 1.5*2^-10 -> nearest of {0, 2^-9} is 2^-9 -> 0x01
    #   2^-17 -> 2^-10 = exact midpoint of 0 and 2^-9 -> even -> 0x00
    x = np.zeros(128, np.float32)
    x[:10] = [1.0, -2.0, 0.5, 3.5, 0.0, -0.0, 0.01171875, 2.0 ** -16, 3 * 2.0 ** -18, 2.0 ** -17]
    codes, s = O.quant_fp8(x[None])
    assert s[0] == np.float32(2.0 ** -7)
    assert codes[0, :10].tolist() == [0x70, 0xF8, 0x68, 0x7E, 0x00, 0x80, 0x3C, 0x01, 0x01, 0x00]
    assert np.all(codes[0, 10:] == 0)


def test_quant_amax_element_maps_to_448():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((500, 128)).astype(np.float32) * rng.uniform(1e-3, 1e3, size=(500, 1)).astype(np.float32)
    codes, s = O.quant_fp8(x)
    i = np.argmax(np.abs(x), axis=1)
    c = codes[np.arange(500), i]
    assert np.all((c == 0x7E) | (c == 0xFE))
    assert np.all(((c >> 7) == 1) == (x[np.arange(500), i] < 0))


def test_quant_zero_and_tiny_rows_use_unit_scale():
    x = np.zeros((3, 128), np.float32)
    x[1, 5] = -(2.0 ** -110)
    x[2, 7] = 2.0 ** -99          # above the 2^-100 threshold: ordinary scale
    codes, s = O.quant_fp8(x)
    assert s[0] == 1.0 and s[1] == 1.0
    assert np.all(codes[0] == 0)
    assert codes[1, 5] == 0x80 and np.count_nonzero(codes[1]) == 1
    assert s[2] == np.float32(np.float32(2.0 ** -99) / np.float32(448.0))
    assert codes[2, 7] == 0x7E


def test_quant_dequant_error_within_half_step():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((300, 128)).astype(np.float32)
    codes, s = O.quant_fp8(x)
    y = x.astype(np.float64) / s[:, None].astype(np.float64)
    d = O.e4m3_decode(codes)
    # half a quantisation step: 2^(e-4) for |y| in [2^e, 2^(e+1)), or 2^-10 for subnormals
    e = np.floor(np.log2(np.maximum(np.abs(y), 2.0 ** -6)))
    bound = np.exp2(e - 4) * (1 + 1e-6) + 1e-7 * np.abs(y)
    assert np.all(np.abs(d - y) <= bound)


def test_bf16_decode_every_pattern_matches_torch():
    # all 65,536 bf16 bit patterns against torch's own bfloat16 -> float64 conversion
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    ours = O.bf16_bits_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert nan.sum() == 2 * 127                 # exponent all ones, non-zero mantissa, both signs
    assert np.array_equal(ours[~nan].view(np.uint64), ref[~nan].view(np.uint64))   # -0 kept
    assert np.array_equal(O.bf16_bits_to_f32(bits)[~nan].astype(np.float64), ref[~nan])
    # a few values fixed by the format: sign, 8 exponent bits (bias 127), 7 mantissa bits
    assert ours[0x3F80] == 1.0 and ours[0xBF80] == -1.0 and ours[0x4049] == 3.140625
    assert ours[0x0001] == 2.0 ** -133 and ours[0x7F7F] == (2 - 2.0 ** -7) * 2.0 ** 127
    assert np.isinf(ours[0x7F80]) and ours[0xFF80] == -np.inf


def test_bf16_round_matches_torch():
    # torch's float32 -> bfloat16 conversion rounds to nearest even: every bf16
    # midpoint and its float32 neighbours, plus random float32 over a wide range
    rng = np.random.default_rng(11)
    b = np.arange(0, 0x7F7F, dtype=np.uint32)                    # finite bf16 magnitudes
    mids = ((b << 16) | 0x8000).view(np.float32)
    cand = [mids, np.nextafter(mids, np.float32(0)), np.nextafter(mids, np.float32(np.inf)),
            ((b << 16)).view(np.float32),
            (rng.standard_normal(1 << 18) * np.exp(rng.uniform(-80, 80, 1 << 18))).astype(np.float32)]
    x = np.concatenate(cand).astype(np.float32)
    x = x[np.isfinite(x) & (np.abs(x) < np.float32(3.38e38))]
    x = np.concatenate([x, -x])
    ours = O.bf16_round(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    bad = np.flatnonzero(ours != ref)
    assert bad.size == 0, (x[bad[:5]], ours[bad[:5]], ref[bad[:5]])
    # ties go to the even mantissa: 1 + 2^-8 lies halfway between 1 and 1 + 2^-7
    assert O.bf16_round(np.float32(1 + 2.0 ** -8))[()] == 0x3F80
    assert O.bf16_round(np.float32(1 + 3 * 2.0 ** -8))[()] == 0x3F82
    assert O.bf16_round(np.float32(-0.0))[()] == 0x8000
