"""Pins for the oracle's multi-axis RoPE.

Closed forms fix the frequencies and the axis split (hand-derived constants:
theta**(-2j/d) for chosen j gives 1, 0.1, 0.01), invariants fix the rotation
itself (identity at zero, norm preservation, composition, relative-position
invariance), and a complex-number formulation gives an independent route.
"""

import math

import numpy as np
import pytest

import oracle

DIMS = (32, 48, 48)
OFF = (0, 32, 80)


def _unit(d):
    x = np.zeros((1, 1, 128))
    x[0, 0, d] = 1.0
    return x


def test_identity_at_zero_bitwise():
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 3, 128))
    y = oracle.rope(x, np.zeros((7, 3)))
    assert np.array_equal(x, y)


@pytest.mark.parametrize(
    "axis,j,omega",
    [
        (0, 0, 1.0),     # t chunk, first pair: theta**0
        (0, 4, 0.1),     # 10000**(-8/32)  = 10**-1
        (0, 8, 0.01),    # 10000**(-16/32) = 10**-2
        (0, 12, 0.001),  # 10000**(-24/32) = 10**-3
        (1, 0, 1.0),
        (1, 6, 0.1),     # 10000**(-12/48)
        (1, 12, 0.01),   # 10000**(-24/48)
        (2, 0, 1.0),
        (2, 18, 0.001),  # 10000**(-36/48)
    ],
)
def test_pair_rotation_closed_form(axis, j, omega):
    # e_{2j} of the chosen chunk at position p on that axis turns to (cos p w, sin p w)
    for p in (1.0, 3.0, 17.0, 41.96875):
        pos = np.zeros((1, 3))
        pos[0, axis] = p
        d = OFF[axis] + 2 * j
        y = oracle.rope(_unit(d), pos)[0, 0]
        expect = np.zeros(128)
        expect[d] = math.cos(p * omega)
        expect[d + 1] = math.sin(p * omega)
        np.testing.assert_allclose(y, expect, rtol=0, atol=1e-14)
        y2 = oracle.rope(_unit(d + 1), pos)[0, 0]
        expect2 = np.zeros(128)
        expect2[d] = -math.sin(p * omega)
        expect2[d + 1] = math.cos(p * omega)
        np.testing.assert_allclose(y2, expect2, rtol=0, atol=1e-14)


def test_axis_chunks_are_separate():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 2, 128))
    for axis in range(3):
        pos = np.zeros((5, 3))
        pos[:, axis] = rng.uniform(1, 40, size=5)
        y = oracle.rope(x, pos)
        lo, hi = OFF[axis], OFF[axis] + DIMS[axis]
        outside = np.ones(128, bool)
        outside[lo:hi] = False
        assert np.array_equal(y[:, :, outside], x[:, :, outside])
        assert not np.allclose(y[:, :, lo:hi], x[:, :, lo:hi])


def test_audio_rows_rotate_on_t_only():
    rng = np.random.default_rng(2)
    x = rng.standard_normal((4, 2, 128))
    pos = np.zeros((4, 3))
    pos[:, 0] = [0.0, 0.03125, 5.5, 31.96875]
    y = oracle.rope(x, pos)
    assert np.array_equal(y[:, :, 32:], x[:, :, 32:])


def test_pair_norms_preserved():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((9, 2, 128))
    pos = rng.uniform(0, 50, size=(9, 3))
    y = oracle.rope(x, pos)
    nx = x[..., 0::2] ** 2 + x[..., 1::2] ** 2
    ny = y[..., 0::2] ** 2 + y[..., 1::2] ** 2
    np.testing.assert_allclose(ny, nx, rtol=1e-13, atol=0)


def test_composition():
    rng = np.random.default_rng(4)
    x = rng.standard_normal((6, 2, 128))
    a = rng.uniform(0, 20, size=(6, 3))
    b = rng.uniform(0, 20, size=(6, 3))
    np.testing.assert_allclose(oracle.rope(oracle.rope(x, a), b), oracle.rope(x, a + b), rtol=0, atol=1e-12)


def test_relative_position_invariance():
    rng = np.random.default_rng(5)
    q = rng.standard_normal((8, 1, 128))
    k = rng.standard_normal((8, 1, 128))
    pos = rng.uniform(0, 40, size=(8, 3))
    shift = np.array([[3.25, -7.0, 11.5]])
    d1 = oracle.rope(q, pos)[:, 0] @ oracle.rope(k, pos)[:, 0].T
    d2 = oracle.rope(q, pos + shift)[:, 0] @ oracle.rope(k, pos + shift)[:, 0].T
    np.testing.assert_allclose(d2, d1, rtol=0, atol=1e-12)


def test_complex_formulation():
    # (x0 + i x1) * exp(i phi), per pair, with textbook complex arithmetic
    rng = np.random.default_rng(6)
    x = rng.standard_normal((5, 2, 128))
    pos = rng.uniform(0, 40, size=(5, 3))
    y = oracle.rope(x, pos)
    z = x[..., 0::2] + 1j * x[..., 1::2]          # [5, 2, 64]
    phase = np.empty((5, 64))
    col = 0
    for axis, width in enumerate(DIMS):
        for j in range(width // 2):
            phase[:, col] = pos[:, axis] * 10000.0 ** (-2.0 * j / width)
            col += 1
    zr = z * np.exp(1j * phase)[:, None, :]
    np.testing.assert_allclose(y[..., 0::2], zr.real, rtol=0, atol=1e-13)
    np.testing.assert_allclose(y[..., 1::2], zr.imag, rtol=0, atol=1e-13)


def test_frequencies_closed_form():
    np.testing.assert_allclose(oracle.rope_frequencies(10000.0, 32)[[0, 4, 8, 12]], [1, 0.1, 0.01, 0.001], rtol=1e-15)
    np.testing.assert_allclose(oracle.rope_frequencies(10000.0, 48)[[0, 6, 12, 18]], [1, 0.1, 0.01, 0.001], rtol=1e-15)
    assert len(oracle.rope_frequencies(10000.0, 48)) == 24
