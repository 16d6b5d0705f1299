"""Oracle query preparation (RoPE + Hadamard, [ATOM-1507] "Where") and the rotation
consistency rule behind the pages' recall bug ([ATOM-1507] "Root cause found": the
index query was Hadamard-rotated while the index key was not).

Pins: a per-vector brute force of the chain, the identities (Hq).(Hk) = q.k and
(Hq).k = q.(Hk) for the orthogonal, symmetric H, and RoPE's dependence on relative
position only.  The rotation-consistency test then shows the failure mode on the
pages' synthetic setting: with consistent rotations a planted needle of a typical
key's length ranks first, with the asymmetric pairing it falls out of the top-k,
while a needle four times longer survives either way (the "artificially strong
needle" of [HYPOTHESIS] "The Context" that hid the bug from the synthetic test)."""
import numpy as np
import pytest

from oracle import oracle as O
from synth import gen

ALL = O.STORE_ROPE | O.STORE_HADAMARD


def _bits(x):
    return gen.f32_to_bf16_bits(np.asarray(x, np.float32))


def test_q_prep_is_the_per_vector_chain():
    rng = np.random.default_rng(1)
    rows, heads = 3, 2
    qb = _bits(rng.normal(size=(rows, heads, 128)))
    pos = rng.integers(0, 1 << 20, size=rows)
    got = O.q_prep(qb, pos, ALL, 10000.0, 64)
    for r in range(rows):
        for h in range(heads):
            x = O.bf16_bits_to_f64(qb[r, h])
            c = O.rope(x[None], [pos[r]], 10000.0, 64)[0]
            ref = np.array([sum(O.hadamard_matrix()[i, j] * c[j] for j in range(128)) for i in range(128)])
            np.testing.assert_allclose(got[r, h], ref / np.sqrt(128.0), rtol=0, atol=1e-12)


def test_q_prep_flags_zero_is_the_decoded_input():
    rng = np.random.default_rng(2)
    qb = _bits(rng.normal(size=(2, 4, 128)))
    assert np.array_equal(O.q_prep(qb, [3, 4], 0, 10000.0, 64), O.bf16_bits_to_f64(qb))


def test_rotation_identities():
    rng = np.random.default_rng(3)
    q = rng.normal(size=(64, 128))
    k = rng.normal(size=(300, 128))
    H = O.hadamard_matrix().astype(np.float64) / np.sqrt(128.0)
    np.testing.assert_allclose((q @ H.T) @ (k @ H.T).T, q @ k.T, rtol=0, atol=1e-10)   # (Hq).(Hk) = q.k
    np.testing.assert_allclose((q @ H.T) @ k.T, q @ (k @ H.T).T, rtol=0, atol=1e-10)   # H symmetric
    assert np.max(np.abs((q @ H.T) @ k.T - q @ k.T)) > 1.0                              # (Hq).k != q.k


def test_rope_depends_on_relative_position_only():
    rng = np.random.default_rng(4)
    qb = _bits(rng.normal(size=(1, 1, 128)))
    kb = _bits(rng.normal(size=(1, 1, 128)))
    def dot(m, n):
        a = O.q_prep(qb, [m], O.STORE_ROPE, 10000.0, 64)[0, 0]
        b = O.q_prep(kb, [n], O.STORE_ROPE, 10000.0, 64)[0, 0]
        return a @ b
    ref = dot(1000, 900)
    for shift in (1, 37, 12345, 600000):
        assert abs(dot(1000 + shift, 900 + shift) - ref) < 1e-9 * max(1.0, abs(ref))
    assert abs(dot(1000, 901) - ref) > 1e-6


@pytest.mark.parametrize("S", [4500, 22000])
def test_rotation_consistency_decides_needle_recall(S):
    k = 512
    wl = gen.make([S], key_dtype="bf16", k=k, seed=0, needle_depth=None)
    keys = O.bf16_bits_to_f64(wl.keys_bits[0])[:S].copy()
    q = O.bf16_bits_to_f64(wl.q_bits[0])
    w = wl.w[0].astype(np.float64)
    H = O.hadamard_matrix().astype(np.float64) / np.sqrt(128.0)
    v = (w[:, None] * q).sum(0)
    typical = np.median(np.linalg.norm(keys, axis=1))
    p = S // 2
    for strength, lost_when_asymmetric in ((1.0, True), (4.0, False)):
        kk = keys.copy()
        kk[p] = strength * typical * v / np.linalg.norm(v)
        consistent = O.score(q @ H.T, w, kk @ H.T)     # both sides rotated
        asymmetric = O.score(q @ H.T, w, kk)           # the pages' bug: the key is not
        assert O.rank_of(consistent, S, p) == 1
        r_bad = O.rank_of(asymmetric, S, p)
        if lost_when_asymmetric:
            assert r_bad > k, r_bad
        else:
            assert r_bad == 1
