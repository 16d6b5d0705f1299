"""Pins of the oracle's score, top-k and Jaccard against exact-rational brute force,
closed forms, invariants, library routines and the values printed on the pages."""
import itertools
import json
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import oracle as O
from synth import gen

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ---------------------------------------------------------------- score ----------

def _bf16(x):
    return O.bf16_bits_to_f64(gen.f32_to_bf16_bits(np.asarray(x, np.float32)))


def test_score_exact_rational_bruteforce():
    rng = np.random.default_rng(0)
    H, S = 3, 7
    q = _bf16(rng.standard_normal((H, 128)))
    k = _bf16(rng.standard_normal((S, 128)))
    w = rng.random(H).astype(np.float32).astype(np.float64) - 0.3      # includes a negative weight
    got = O.score(q, w, k)
    for p in range(S):
        tot = Fraction(0)
        for h in range(H):
            dot = sum(Fraction(float(q[h, d])) * Fraction(float(k[p, d])) for d in range(128))
            tot += Fraction(float(w[h])) * max(dot, Fraction(0))
        assert abs(got[p] - float(tot)) <= 1e-15 * max(1.0, abs(float(tot)))


def test_score_closed_forms():
    H = 4
    w = np.array([0.5, 0.25, 2.0, 1.0])
    # one-hot q (head h on dim h) against one-hot keys: score = w_h if key dim == h
    q = np.zeros((H, 128))
    q[np.arange(H), np.arange(H)] = 1.0
    keys = np.zeros((6, 128))
    keys[np.arange(6), np.arange(6)] = 1.0
    assert np.array_equal(O.score(q, w, keys), np.array([0.5, 0.25, 2.0, 1.0, 0.0, 0.0]))
    rng = np.random.default_rng(1)
    kt = rng.standard_normal((1, 128))
    # q_h = k_t for every head: sum_h w_h ||k_t||^2
    assert math.isclose(O.score(np.repeat(kt, H, 0), w, kt)[0], w.sum() * float((kt @ kt.T).item()), rel_tol=1e-14)
    # q_h = -k_t: every logit negative, ReLU gives exactly zero
    assert O.score(np.repeat(-kt, H, 0), w, kt)[0] == 0.0


def test_score_mask_ignores_keys_beyond_row_len():
    rng = np.random.default_rng(2)
    q, w = rng.standard_normal((8, 128)), rng.random(8)
    keys = rng.standard_normal((50, 128))
    poisoned = keys.copy()
    poisoned[30:] = np.nan
    assert np.array_equal(O.score(q, w, poisoned, 30), O.score(q, w, keys[:30]))
    m = O.score_rows(q[None], w[None], [poisoned], [0], [30], 50)
    assert np.all(np.isneginf(m[0, 30:])) and np.array_equal(m[0, :30], O.score(q, w, keys[:30]))


def test_score_invariances():
    rng = np.random.default_rng(3)
    q, w = rng.standard_normal((16, 128)), rng.random(16)
    keys = rng.standard_normal((40, 128))
    base = O.score(q, w, keys)
    perm = rng.permutation(16)
    assert np.allclose(O.score(q[perm], w[perm], keys), base, rtol=1e-13)     # heads commute
    assert np.array_equal(O.score(q, 4.0 * w, keys), 4.0 * base)              # homogeneous in w
    assert np.array_equal(O.score(q, w, keys * 0.125), base * 0.125)          # key scale factors out
    s = 0.0137
    assert np.allclose(O.score(q, w, keys * s), base * s, rtol=1e-13)


def test_score_fp8_keys_scale_factorisation():
    # per-key scale applied after the head sum equals scoring the dequantised keys
    rng = np.random.default_rng(4)
    x = rng.standard_normal((30, 128)).astype(np.float32)
    codes, s = O.quant_fp8(x)
    q, w = rng.standard_normal((8, 128)), rng.random(8)
    a = O.score(q, w, O.dequant_fp8(codes, s))
    b = O.score(q, w, O.e4m3_decode(codes)) * s.astype(np.float64)
    assert np.allclose(a, b, rtol=1e-13)


def _needle_case(S, key_dtype):
    wl = gen.make([S], key_dtype=key_dtype, k=512, needle_depth=(0.4, 0.6), seed=0, shuffle=False)
    q = O.bf16_bits_to_f64(wl.q_bits[0])
    x = wl.keys_bits[0]
    if key_dtype == "fp8":
        keys = O.dequant_fp8(*O.quant_fp8(O.bf16_bits_to_f32(x)))
    else:
        keys = O.bf16_bits_to_f64(x)
    sc = O.score(q, wl.w[0].astype(np.float64), keys)
    return wl, sc


def test_needle_ranks_first_like_the_printed_table():
    table = json.load(open(os.path.join(GOLDEN, "synthetic_fp8_vs_bf16_top512.json")))
    for row in table["rows"]:
        sel = {}
        for dt in ("bf16", "fp8"):
            wl, sc = _needle_case(row["S"], dt)
            p = int(wl.needle_pos[0])
            assert O.rank_of(sc, sc.size, p) == row[f"rank_{dt}"] == 1
            sel[dt] = O.topk(sc[None], [sc.size], 512)
            assert p in set(sel[dt][0].tolist())
        j, lost = O.jaccard(sel["bf16"], sel["fp8"])
        assert 0.0 < j < 1.0 and 0 < lost < 512


# ---------------------------------------------------------------- top-k ----------

def _brute_topk(vals, k):
    n = len(vals)
    best, best_set = None, None
    for comb in itertools.combinations(range(n), min(k, n)):       # lexicographic order
        s = sum(vals[i] for i in comb)
        if best is None or s > best:
            best, best_set = s, comb
    return list(best_set)


def test_topk_subset_bruteforce_with_ties():
    rng = np.random.default_rng(0)
    for trial in range(60):
        n = int(rng.integers(1, 10))
        vals = rng.integers(-3, 4, size=n).astype(np.float64)     # many ties, exact sums
        for k in range(1, n + 2):
            got = O.topk(vals[None], [n], k)[0]
            want = _brute_topk(vals.tolist(), k)
            assert got[:len(want)].tolist() == want
            assert np.all(got[len(want):] == -1)


def test_topk_special_cases():
    eq = np.full((1, 100), 2.5)
    assert O.topk(eq, [100], 10)[0].tolist() == list(range(10))            # tie-break: lowest index
    inc = np.arange(100, dtype=np.float64)[None]
    assert O.topk(inc, [100], 5)[0].tolist() == [95, 96, 97, 98, 99]
    assert O.topk(inc, [60], 5)[0].tolist() == [55, 56, 57, 58, 59]         # causal cut
    r = O.topk(inc, [3], 5)[0].tolist()
    assert r == [0, 1, 2, -1, -1]                                           # k >= row_len: all, padded
    assert O.topk(inc, [0], 4)[0].tolist() == [-1, -1, -1, -1]
    z = np.array([[0.0, -0.0, 1.0, -0.0, 0.0]])
    assert O.topk(z, [5], 3)[0].tolist() == [0, 1, 2]                       # -0 == +0


def test_topk_matches_torch_topk_on_distinct_values():
    rng = np.random.default_rng(1)
    x = rng.permutation(50000).astype(np.float64).reshape(5, 10000) * 0.5
    lens = [10000, 9000, 5000, 1025, 1024]
    got = O.topk(x, lens, 1024)
    for r in range(5):
        t = torch.topk(torch.from_numpy(x[r, :lens[r]]), min(1024, lens[r])).indices.numpy()
        assert np.array_equal(np.sort(t), got[r, :t.size])


def _nan_f32(bits):
    return np.array([bits], dtype=np.uint32).view(np.float32)[0]


def test_topk_nan_order_matches_torch_topk():
    # NaNs of both signs and several payloads rank above +inf, as in torch.topk
    nans = [_nan_f32(b) for b in (0x7FC00000, 0xFFC00000, 0x7F800001, 0xFFFFFFFF)]
    rng = np.random.default_rng(2)
    for trial in range(20):
        n = int(rng.integers(8, 400))
        x = (rng.permutation(n).astype(np.float32) - n / 2) * np.float32(0.25)
        m = int(rng.integers(1, min(n, 12)))
        at = rng.choice(n, m, replace=False)
        x[at] = [nans[i % 4] for i in range(m)]
        x[rng.integers(n)] = np.float32(np.inf) if m < n else x[0]
        for k in (m, m + 1, min(n, m + 7)):
            got = O.topk(x[None], [n], k)[0]
            t = torch.topk(torch.from_numpy(x), k).indices.numpy()
            assert np.array_equal(np.sort(t), got[:k]), (trial, k)
    # worked row: NaNs first, then +inf, then the largest numbers; NaNs tie by position
    row = np.array([1.0, nans[1], 3.0, np.inf, nans[0], -np.inf, nans[2]], dtype=np.float32)
    assert O.topk(row[None], [7], 4)[0].tolist() == [1, 3, 4, 6]
    assert O.topk(row[None], [7], 2)[0].tolist() == [1, 4]
    assert O.topk(row[None], [7], 5)[0].tolist() == [1, 2, 3, 4, 6]
    assert O.topk(row[None], [6], 7)[0].tolist() == [0, 1, 2, 3, 4, 5, -1]


# ---------------------------------------------------------------- jaccard --------

def test_jaccard_reproduces_printed_table():
    table = json.load(open(os.path.join(GOLDEN, "synthetic_fp8_vs_bf16_top512.json")))
    k = table["k"]
    for row in table["rows"]:
        lost = row["lost"]
        a = np.arange(k)
        b = np.concatenate([np.arange(lost, k), np.arange(10000, 10000 + lost)])   # |A\B| = lost
        j, l2 = O.jaccard(a, b)
        assert l2 == lost
        assert round(j, 3) == row["jaccard"]
        assert math.isclose(j, (k - lost) / (k + lost))


def test_jaccard_ignores_padding():
    assert O.jaccard([1, 2, -1], [2, 1, -1]) == (1.0, 0)
    assert O.jaccard([1, 2, 3, -1], [2, 5, -1, -1]) == (0.25, 2)


# ---------------------------------------------------------------- threshold ------

def test_kth_score_hand_worked_row_with_ties():
    # descending order of the first 7 entries: 9, 7, 7, 7, 4, 1, -2 (the 8th entry is
    # past the visible length and must not count)
    row = np.array([7.0, 1.0, 9.0, 7.0, -2.0, 4.0, 7.0, 100.0])
    n = 7
    assert [O.kth_score(row, n, k) for k in range(1, 8)] == [9.0, 7.0, 7.0, 7.0, 4.0, 1.0, -2.0]
    # k >= n: the smallest visible score
    assert O.kth_score(row, n, 7) == O.kth_score(row, n, 8) == O.kth_score(row, n, 1000) == -2.0
    # the threshold is the score of the last element the oracle's top-k keeps
    for k in range(1, 8):
        keep = O.topk(row[None], [n], k)[0][:k]
        assert min(row[keep]) == O.kth_score(row, n, k)


def test_kth_score_is_the_kth_order_statistic():
    # against a counting definition: tau has >= k visible scores at or above it and
    # fewer than k strictly above it
    rng = np.random.default_rng(5)
    for trial in range(200):
        n = int(rng.integers(1, 40))
        row = rng.integers(-4, 5, size=n + 3).astype(np.float64)
        for k in range(1, n + 3):
            t = O.kth_score(row, n, k)
            vis = row[:n]
            kk = min(k, n)
            assert np.sum(vis >= t) >= kk and np.sum(vis > t) < kk
