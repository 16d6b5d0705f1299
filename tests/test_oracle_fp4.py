"""Pins of the oracle's MXFP4 (e2m1 + e8m0 per 32) index-key quantiser.

The e2m1 value table is the OCP format's (from its exponent/mantissa definition);
rounding is checked against exact rational nearest-value search; the block
exponent against its defining inequality, with the element error bound and a
hand-worked block.  (torch has an e2m1 dtype but no conversion into it here.)"""
from fractions import Fraction

import numpy as np
import pytest

from oracle import oracle as O


def test_e2m1_values_of_the_format():
    # OCP MX: e2m1, exponent bias 1; subnormal m * 0.5; normals 2^(e-1) * (1 + m/2)
    want = []
    for e in range(4):
        for m in range(2):
            want.append(0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + m / 2))
    assert want == [0, 0.5, 1, 1.5, 2, 3, 4, 6]
    assert np.array_equal(O.e2m1_decode(np.arange(8)), want)
    assert np.array_equal(O.e2m1_decode(np.arange(8, 16)), [-x for x in want])
    # every code round-trips (except -0, whose value is 0 but whose code keeps the sign)
    assert np.array_equal(O.e2m1_encode(O.e2m1_decode(np.arange(16))), np.arange(16))


def test_e2m1_rounding_brute_force():
    # exact nearest magnitude with ties to the even mantissa bit, on a fine rational
    # grid that hits every tie, plus random reals; saturation beyond 6
    mags = [Fraction(x) for x in (0, 0.5, 1, 1.5, 2, 3, 4, 6)]

    def want(x):
        a = abs(Fraction(x))
        if a > 6:
            c = 7
        else:
            best = min(range(8), key=lambda i: (abs(mags[i] - a), i % 2))
            c = best
        return c | (8 if np.signbit(x) else 0)

    grid = np.array([k / 16 for k in range(-8 * 16, 8 * 16 + 1)] + [-0.0])
    rnd = np.random.default_rng(0).uniform(-9, 9, 2000)
    for v in np.concatenate([grid, rnd]):
        assert O.e2m1_encode(v) == want(v), v
    # the ties by name: 0.25 -> 0, 0.75 -> 1, 1.25 -> 1, 1.75 -> 2, 2.5 -> 2, 3.5 -> 4, 5 -> 4
    ties = O.e2m1_decode(O.e2m1_encode([0.25, 0.75, 1.25, 1.75, 2.5, 3.5, 5.0]))
    assert np.array_equal(ties, [0, 1, 1, 2, 2, 4, 4])


def test_block_exponent_inequality_and_error_bound():
    rng = np.random.default_rng(1)
    x = (rng.standard_normal((200, 128)) * np.exp(rng.uniform(-30, 30, (200, 1)))).astype(np.float32)
    x[0, :32] = 0.0                               # an all-zero block
    x[1, 32:64] = np.float32(2.0 ** -140)         # a block limited by the e8m0 range
    codes, e8 = O.quant_mxfp4(x)
    assert codes.shape == x.shape and e8.shape == (200, 4)
    assert e8[0, 0] == 127 and np.all(codes[0, :32] == 0)
    e = e8.astype(np.int64) - 127
    amax = np.abs(x.astype(np.float64)).reshape(200, 4, 32).max(-1)
    live = (amax > 0) & (e > -127)
    # defining inequality: 2^(e+2) <= amax < 2^(e+3)
    assert np.all(np.ldexp(1.0, e + 2)[live] <= amax[live])
    assert np.all(amax[live] < np.ldexp(1.0, e + 3)[live])
    assert e[1, 1] == -127
    # error bound: half a step of the e2m1 grid at the element's magnitude, or the
    # saturation excess beyond 6 * 2^e
    y = O.dequant_mxfp4(codes, e8).reshape(200, 4, 32)
    xb = x.astype(np.float64).reshape(200, 4, 32)
    v = np.abs(xb) / np.ldexp(1.0, e)[..., None]
    step = np.where(v < 2, 0.5, np.where(v < 4, 1.0, 2.0))
    bound = np.where(v > 6, v - 6, step / 2) * np.ldexp(1.0, e)[..., None]
    assert np.all(np.abs(y - xb) <= bound * (1 + 1e-12))
    # the block maximum lands on 4 or 6 times the scale (amax / 2^e in [4, 8))
    top = np.abs(y).max(-1)
    ok = live
    assert np.all(np.isin(top[ok] / np.ldexp(1.0, e)[ok], [4.0, 6.0]))


def test_hand_worked_block():
    # amax 10 -> floor(log2 10) = 3 -> e = 1, scale 2: values / 2 rounded to e2m1
    x = np.zeros(128, np.float32)
    x[:8] = [10.0, -3.0, 0.5, 0.49, 2.5, 7.0, -12.5, 0.0]
    codes, e8 = O.quant_mxfp4(x)
    assert e8[0] == 128
    # 10/2 = 5 -> tie 4|6 -> 4 (code 6); -1.5 (11); 0.25 -> tie 0|0.5 -> 0 (0);
    # 0.245 -> 0 (0); 1.25 -> tie 1|1.5 -> 1 (2); 3.5 -> tie 3|4 -> 4 (6);
    # -6.25 -> saturates to -6 (15); 0 (0)
    assert list(codes[:8]) == [6, 11, 0, 0, 2, 6, 15, 0]
    assert np.all(codes[8:32] == 0) and list(e8[1:]) == [127, 127, 127]
