"""Pins of the oracle's store chain (RMSNorm -> RoPE -> Hadamard) against closed
forms, invariants and a library routine."""
import cmath
import math

import numpy as np
import scipy.linalg

from oracle import oracle as O
from synth import gen


def test_hadamard_closed_form_and_library():
    h = O.hadamard_matrix(128)
    i = np.arange(128)
    # Sylvester order: H[i, j] = (-1)^popcount(i & j)
    pc = np.vectorize(lambda v: bin(int(v)).count("1"))(i[:, None] & i[None, :])
    assert np.array_equal(h, (-1) ** pc)
    assert np.array_equal(h, scipy.linalg.hadamard(128))
    assert np.array_equal(h @ h.T, 128 * np.eye(128, dtype=np.int64))


def _fwht(x):
    """Iterative fast Walsh-Hadamard transform (butterflies), independent of the
    oracle's dense Sylvester matrix."""
    x = np.array(x, dtype=np.float64, copy=True)
    n = x.shape[-1]
    hlen = 1
    while hlen < n:
        for s in range(0, n, 2 * hlen):
            a = x[..., s:s + hlen].copy()
            b = x[..., s + hlen:s + 2 * hlen].copy()
            x[..., s:s + hlen] = a + b
            x[..., s + hlen:s + 2 * hlen] = a - b
        hlen *= 2
    return x


def test_hadamard_rotation_orthogonal_and_involution():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((20, 128))
    bits = gen.f32_to_bf16_bits(x.astype(np.float32))
    y = O.store_chain(bits, np.zeros(20), O.STORE_HADAMARD, 1e-6, 10000.0, 64)
    xd = O.bf16_bits_to_f64(bits)
    assert np.allclose(y, _fwht(xd) / math.sqrt(128), rtol=0, atol=1e-13)
    # norm preserved; (Hq).(Hk) = q.k; applying the normalised H twice is the identity
    assert np.allclose(np.linalg.norm(y, axis=1), np.linalg.norm(xd, axis=1), rtol=1e-13)
    assert np.allclose(y[:10] @ y[10:].T, xd[:10] @ xd[10:].T, rtol=1e-12, atol=1e-12)
    hn = O.hadamard_matrix(128) / math.sqrt(128)
    assert np.allclose(hn @ hn, np.eye(128), atol=1e-14)


def test_rope_position_zero_is_identity_and_untouched_dims():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((6, 128))
    y = O.rope(x, np.zeros(6), 10000.0, 64)
    assert np.array_equal(y, x)
    z = O.rope(x, np.arange(6) * 1000 + 7, 10000.0, 64)
    assert np.array_equal(z[:, :64], x[:, :64])       # only the trailing rope_dim rotate


def test_rope_pair_norms_preserved():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((5, 128))
    pos = np.array([0, 1, 77, 65535, 1048575])
    for rd in (2, 32, 64, 128):
        y = O.rope(x, pos, 10000.0, rd)
        o = 128 - rd
        n0 = x[:, o::2] ** 2 + x[:, o + 1::2] ** 2
        n1 = y[:, o::2] ** 2 + y[:, o + 1::2] ** 2
        assert np.allclose(n0, n1, rtol=1e-12)


def test_rope_closed_forms():
    # rope_dim = 2: one pair at the end, angle = pos * base^0 = pos; compare with a
    # complex rotation e^{i pos}
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 128))
    pos = np.array([0, 3, 1000, 1048575])
    y = O.rope(x, pos, 10000.0, 2)
    for r in range(4):
        z = complex(x[r, 126], x[r, 127]) * cmath.exp(1j * float(pos[r]))
        assert abs(complex(y[r, 126], y[r, 127]) - z) < 1e-9
    # rope_dim = 4, base 10000, pos 1: pair 1 has angle 10000^(-1/2) = 0.01
    e = np.zeros((1, 128))
    e[0, 126] = 1.0
    y = O.rope(e, np.array([1]), 10000.0, 4)
    assert abs(y[0, 126] - math.cos(0.01)) < 1e-15 and abs(y[0, 127] - math.sin(0.01)) < 1e-15


def test_rope_relative_position_property_near_1m():
    # <RoPE(q, m), RoPE(k, n)> depends only on m - n, also at positions near 1M
    rng = np.random.default_rng(4)
    q = rng.standard_normal((1, 128))
    k = rng.standard_normal((1, 128))
    for base in (10000.0, 160000.0):
        a = (O.rope(q, [1048000], base, 64) @ O.rope(k, [1047000], base, 64).T).item()
        b = (O.rope(q, [1000], base, 64) @ O.rope(k, [0], base, 64).T).item()
        assert abs(a - b) < 1e-8 * (1 + abs(b))


def test_rmsnorm_unit_rms_and_scale_invariance():
    rng = np.random.default_rng(5)
    x = rng.standard_normal((8, 128)) * 3
    y = O.rmsnorm(x, 0.0)
    assert np.allclose(np.mean(y * y, axis=1), 1.0, rtol=1e-14)
    assert np.allclose(O.rmsnorm(x * 37.5, 0.0), y, rtol=1e-14)
    assert np.array_equal(O.rmsnorm(np.full((1, 128), 2.0), 0.0), np.ones((1, 128)))


def test_store_chain_flags_compose_in_order():
    rng = np.random.default_rng(6)
    bits = gen.f32_to_bf16_bits(rng.standard_normal((3, 128)).astype(np.float32))
    pos = np.array([5, 600, 1048575])
    x = O.bf16_bits_to_f64(bits)
    assert np.array_equal(O.store_chain(bits, pos, 0, 1e-6, 1e4, 64), x)
    full = O.store_chain(bits, pos, 7, 1e-6, 1e4, 64)
    manual = _fwht(O.rope(O.rmsnorm(x, 1e-6), pos, 1e4, 64)) / math.sqrt(128)
    assert np.allclose(full, manual, rtol=0, atol=1e-13)
