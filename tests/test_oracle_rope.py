"""Pins for oracle.rope: complex-multiplication form and relative positions."""

import numpy as np

from oracle import rope as R


def _x(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_matches_complex_multiplication():
    n, h, d, base = 50, 3, 16, 1e4
    x = _x((2, n, h, d), 0)
    z = x[..., 0::2] + 1j * x[..., 1::2]
    p = np.arange(d // 2)
    th = base ** (-2.0 * p / d)
    rot = np.exp(1j * np.arange(n)[:, None, None] * th[None, None, :])
    want = z * rot
    got = R.rotate(x, base)
    assert np.allclose(got[..., 0::2], want.real, atol=1e-12)
    assert np.allclose(got[..., 1::2], want.imag, atol=1e-12)


def test_relative_position_and_norm():
    n, d, base = 40, 8, 1e4
    q = _x((1, n, 1, d), 1)
    k = _x((1, n, 1, d), 2)
    # the same vectors placed at every position
    q = np.repeat(q[:, :1], n, axis=1)
    k = np.repeat(k[:, :1], n, axis=1)
    qr, kr = R.rotate(q, base), R.rotate(k, base)
    for delta in (0, 3, 17):
        dots = [float(qr[0, i, 0] @ kr[0, i - delta, 0]) for i in range(delta, n)]
        assert np.allclose(dots, dots[0], atol=1e-10)
    assert np.allclose(np.linalg.norm(qr, axis=-1), np.linalg.norm(q, axis=-1))


def test_inverse_and_identity():
    x = _x((2, 30, 2, 16), 3)
    assert np.allclose(R.rotate_back(R.rotate(x, 1e4), 1e4), x, atol=1e-12)
    assert np.array_equal(R.rotate(x, 0.0), x)
    # position 0 is never rotated
    assert np.allclose(R.rotate(x, 1e4)[:, 0], x[:, 0])
