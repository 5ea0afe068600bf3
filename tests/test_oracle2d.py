"""Pins of the 2D oracle (oracle/rdfft2d_oracle.py) against things other than
itself (CPU only): a brute-force 2D DFT with the layout written out by hand,
closed forms, the 1D transform of a row-constant array, numpy's rfft2 half
spectrum, round trips, Parseval and the 2D shift theorem.  A swapped Re/Im
slot, a wrong column convention or a dropped conjugation fails one of them."""

import math

import numpy as np
import pytest

from oracle import rdfft2d_oracle as r2
from oracle import rdfft_oracle as ro

SIZES = [(2, 2), (2, 8), (4, 4), (8, 2), (4, 16), (16, 8)]


def brute_dft2(x):
    h, w = x.shape
    y = np.zeros((h, w), dtype=np.complex128)
    for j in range(h):
        for k in range(w):
            acc = 0j
            for n in range(h):
                for m in range(w):
                    # exact reduction of the phase before the angle
                    num = ((j * n) % h) * w + ((k * m) % w) * h
                    ang = 2.0 * math.pi * (num % (h * w)) / (h * w)
                    acc += x[n, m] * complex(math.cos(ang), -math.sin(ang))
            y[j, k] = acc
    return y


def hand_pack(y):
    """the layout, slot by slot, as stated in the oracle's docstring"""
    h, w = y.shape
    z = np.zeros((h, w))
    for k in range(w // 2 + 1):
        if k == 0 or k == w // 2:
            for j in range(h // 2 + 1):
                z[j, k] = y[j, k].real
                if 0 < j < h // 2:
                    z[h - j, k] = y[j, k].imag
        else:
            for j in range(h):
                z[j, k] = y[j, k].real
                z[j, w - k] = y[j, k].imag
    return z


@pytest.mark.parametrize("h,w", SIZES)
def test_bruteforce_layout(h, w):
    x = np.random.default_rng(h * 100 + w).standard_normal((h, w))
    want = hand_pack(brute_dft2(x))
    assert np.allclose(r2.rdfft2d_forward(x), want, atol=1e-11)


@pytest.mark.parametrize("h,w", [(4, 8), (16, 16), (8, 64)])
def test_closed_forms(h, w):
    n = np.arange(h)[:, None]
    m = np.arange(w)[None, :]
    delta = np.zeros((h, w))
    delta[0, 0] = 1
    z = r2.rdfft2d_forward(delta)
    want = np.zeros((h, w))
    for k in (0, w // 2):
        want[: h // 2 + 1, k] = 1.0  # Re slots of the packed columns
    want[:, 1 : w // 2] = 1.0  # Re Y for 0 < k < W/2; Im slots stay 0
    assert np.allclose(z, want, atol=1e-12)
    z = r2.rdfft2d_forward(np.ones((h, w)))
    want = np.zeros((h, w))
    want[0, 0] = h * w
    assert np.allclose(z, want, atol=1e-9)
    # cos along m: Y[0, 1] = Y[0, W-1] = HW/2 -> slot [0, 1]
    z = r2.rdfft2d_forward(np.cos(2 * np.pi * m / w) + 0 * n)
    want = np.zeros((h, w))
    want[0, 1] = h * w / 2
    assert np.allclose(z, want, atol=1e-9)
    # sin along n: Y[1, 0] = -i HW/2 -> column 0 packed, slot [H-1, 0] = Im Y[1, 0]
    z = r2.rdfft2d_forward(np.sin(2 * np.pi * n / h) + 0 * m)
    want = np.zeros((h, w))
    want[h - 1, 0] = -h * w / 2
    assert np.allclose(z, want, atol=1e-9)


@pytest.mark.parametrize("h,w", [(4, 16), (32, 8)])
def test_row_constant_array_is_the_1d_transform(h, w):
    row = np.random.default_rng(7).standard_normal(w)
    z = r2.rdfft2d_forward(np.tile(row, (h, 1)))
    want = np.zeros((h, w))
    want[0] = h * ro.rdfft_forward(row)
    assert np.allclose(z, want, atol=1e-10)


@pytest.mark.parametrize("h,w", [(8, 32), (64, 16), (2, 4)])
def test_matches_numpy_rfft2(h, w):
    x = np.random.default_rng(h + w).standard_normal((3, h, w))
    half = r2.unpack2d(r2.rdfft2d_forward(x))[..., : w // 2 + 1]
    assert np.allclose(half, np.fft.rfft2(x), atol=1e-10)


@pytest.mark.parametrize("h,w", SIZES + [(64, 128)])
def test_roundtrips(h, w):
    g = np.random.default_rng(h * w)
    x = g.standard_normal((2, h, w))
    assert np.allclose(r2.rdfft2d_inverse(r2.rdfft2d_forward(x)), x, atol=1e-12)
    z = g.standard_normal((2, h, w))  # any packed array is a valid spectrum
    assert np.allclose(r2.rdfft2d_forward(r2.rdfft2d_inverse(z)), z, atol=1e-10)


def test_parseval_and_shift():
    h, w = 16, 32
    x = np.random.default_rng(3).standard_normal((h, w))
    y = r2.unpack2d(r2.rdfft2d_forward(x))
    assert math.isclose(float(np.sum(x**2)), float(np.sum(np.abs(y) ** 2)) / (h * w), rel_tol=1e-12)
    a, b = 3, 5
    ys = r2.unpack2d(r2.rdfft2d_forward(np.roll(x, (a, b), axis=(0, 1))))
    j = np.arange(h)[:, None]
    k = np.arange(w)[None, :]
    assert np.allclose(ys, y * np.exp(-2j * np.pi * (j * a / h + k * b / w)), atol=1e-10)


def test_rejects_bad_sizes():
    for shape in ((3, 4), (4, 6), (1, 4)):
        with pytest.raises(ValueError):
            r2.rdfft2d_forward(np.zeros(shape))
