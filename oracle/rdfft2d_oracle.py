"""fp64 oracle for the 2D packed real FFT -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It shares no code with the HIP library.

The pages leave the 2D extension open (Paper-Notes page, "局限与展望": only the
1D transform is done, 2D is future work).  The reading taken here is the
natural in-place one: an H x W real array is replaced, in its own H*W reals,
by its 2D DFT

    Y[j, k] = sum_n sum_m x[n, m] exp(-2 pi i (j n / H + k m / W)),

of which the half k = 0..W/2 determines the rest (Y[H-j, W-k] = conj Y[j, k]).
The H*W reals hold it as follows (the 1D packing rule of the Paper-Notes page,
"Squeeze", applied along each axis where the data is conjugate-symmetric):

  * columns k = 0 and k = W/2: Y[., k] is conjugate-symmetric in j, so column
    k holds its 1D packed form along j: [0, k] = Y[0, k], [H/2, k] = Y[H/2, k]
    (both real), [j, k] = Re Y[j, k] and [H-j, k] = Im Y[j, k], 0 < j < H/2;
  * columns 0 < k < W/2: [j, k] = Re Y[j, k] and [j, W-k] = Im Y[j, k] for
    every j = 0..H-1.

This is the real 2D half spectrum, nothing lost or duplicated.  The DFT is
numpy's complex 2D FFT in float64 (a library primitive standing for the
definition); the forward is unnormalised and the inverse carries 1/(H W).
"""

from __future__ import annotations

import numpy as np

__all__ = ["pack2d", "unpack2d", "rdfft2d_forward", "rdfft2d_inverse"]


def _check(h: int, w: int) -> None:
    for n in (h, w):
        if n < 2 or n & (n - 1):
            raise ValueError(f"sizes must be powers of two >= 2, got {h} x {w}")


def pack2d(y: np.ndarray) -> np.ndarray:
    """Full 2D spectrum (..., H, W) of real arrays -> packed reals (..., H, W)."""
    y = np.asarray(y)
    h, w = y.shape[-2:]
    _check(h, w)
    z = np.empty(y.shape, dtype=np.float64)
    j = np.arange(1, h // 2)
    for k in (0, w // 2):
        z[..., 0, k] = y[..., 0, k].real
        z[..., h // 2, k] = y[..., h // 2, k].real
        z[..., j, k] = y[..., j, k].real
        z[..., h - j, k] = y[..., j, k].imag
    k = np.arange(1, w // 2)
    z[..., :, k] = y[..., :, k].real
    z[..., :, w - k] = y[..., :, k].imag
    return z


def unpack2d(z: np.ndarray) -> np.ndarray:
    """Packed reals (..., H, W) -> full conjugate-symmetric 2D spectrum (..., H, W)."""
    z = np.asarray(z, dtype=np.float64)
    h, w = z.shape[-2:]
    _check(h, w)
    y = np.zeros(z.shape, dtype=np.complex128)
    j = np.arange(1, h // 2)
    for k in (0, w // 2):
        y[..., 0, k] = z[..., 0, k]
        y[..., h // 2, k] = z[..., h // 2, k]
        y[..., j, k] = z[..., j, k] + 1j * z[..., h - j, k]
        y[..., h - j, k] = z[..., j, k] - 1j * z[..., h - j, k]
    k = np.arange(1, w // 2)
    half = z[..., :, k] + 1j * z[..., :, w - k]  # Y[j, k] for every j
    y[..., :, k] = half
    # Y[j, W-k] = conj Y[(H-j) mod H, k]
    jm = (-np.arange(h)) % h
    y[..., :, w - k] = np.conj(half[..., jm, :])
    return y


def rdfft2d_forward(x: np.ndarray) -> np.ndarray:
    """Packed 2D forward transform of the last two axes, float64."""
    x = np.asarray(x, dtype=np.float64)
    _check(*x.shape[-2:])
    return pack2d(np.fft.fft2(x, axes=(-2, -1)))


def rdfft2d_inverse(z: np.ndarray) -> np.ndarray:
    """Inverse of :func:`rdfft2d_forward` (carries 1/(H W)), float64."""
    y = unpack2d(z)
    return np.ascontiguousarray(np.fft.ifft2(y, axes=(-2, -1)).real)
