"""fp64 oracle for the packed real FFT (rdFFT) -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It shares no code with the HIP library.

What is computed (plain definitions, no blocking or reordering):

* Forward transform of a real row x of length r (r a power of two, r >= 2):
  the DFT  y_k = sum_n x_n exp(-2 pi i k n / r),  written into r reals with the
  pages' packing rule (Paper-Notes page, "关键设计 / Squeeze"; scime.ai page,
  "Approach"): y_0 at index 0, y_{r/2} at index r/2, Re y_k at index k and
  Im y_k at index r-k for 0 < k < r/2.  Both y_0 and y_{r/2} are real and
  y_{r-k} = conj(y_k), so nothing is lost.  The DFT itself is taken from
  numpy's complex FFT in float64 (a library primitive standing for the
  definition); the forward is unnormalised.
* Inverse transform: unpack the r reals into the conjugate-symmetric spectrum
  and apply the inverse DFT with the 1/r factor (the pages halve at every
  inverse stage, Paper-Notes page, "原地 IFFT 设计"; log2 r halvings = 1/r).
* Packed product: the element-wise product of two spectra (optionally the
  first conjugated), packed again; the pages note that such products stay
  conjugate-symmetric (Paper-Notes page, "循环矩阵训练适配").

Readings taken where the pages are silent: the forward exponent sign is
negative (the torch.fft / numpy convention of the pages' baselines), the
forward is unnormalised and the inverse carries 1/r.
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "is_pow2",
    "pack_spectrum",
    "unpack_spectrum",
    "rdfft_forward",
    "rdfft_inverse",
    "packed_product",
]


def is_pow2(r: int) -> bool:
    return r >= 2 and (r & (r - 1)) == 0


def _check_len(r: int) -> None:
    if not is_pow2(r):
        raise ValueError(f"row length must be a power of two >= 2, got {r}")


def pack_spectrum(y: np.ndarray) -> np.ndarray:
    """Full complex spectrum (..., r) of real rows -> packed reals (..., r).

    Slot rule (Paper-Notes page, "Squeeze"): [0] = y_0, [r/2] = y_{r/2},
    [k] = Re y_k and [r-k] = Im y_k for 0 < k < r/2.
    """
    y = np.asarray(y)
    r = y.shape[-1]
    _check_len(r)
    z = np.empty(y.shape, dtype=np.float64)
    z[..., 0] = y[..., 0].real
    z[..., r // 2] = y[..., r // 2].real
    k = np.arange(1, r // 2)
    z[..., k] = y[..., k].real
    z[..., r - k] = y[..., k].imag
    return z


def unpack_spectrum(z: np.ndarray) -> np.ndarray:
    """Packed reals (..., r) -> full conjugate-symmetric complex spectrum (..., r)."""
    z = np.asarray(z, dtype=np.float64)
    r = z.shape[-1]
    _check_len(r)
    y = np.zeros(z.shape, dtype=np.complex128)
    y[..., 0] = z[..., 0]
    y[..., r // 2] = z[..., r // 2]
    k = np.arange(1, r // 2)
    y[..., k] = z[..., k] + 1j * z[..., r - k]
    y[..., r - k] = z[..., k] - 1j * z[..., r - k]
    return y


def rdfft_forward(x: np.ndarray) -> np.ndarray:
    """Packed forward transform of every row of ``x`` (last axis), float64."""
    x = np.asarray(x, dtype=np.float64)
    _check_len(x.shape[-1])
    return pack_spectrum(np.fft.fft(x, axis=-1))


def rdfft_inverse(z: np.ndarray) -> np.ndarray:
    """Inverse of :func:`rdfft_forward` (carries the 1/r factor), float64."""
    y = unpack_spectrum(z)
    x = np.fft.ifft(y, axis=-1)
    return np.ascontiguousarray(x.real)


def packed_product(a: np.ndarray, b: np.ndarray, conj_a: bool = False) -> np.ndarray:
    """Packed spectrum of the bin-wise product a_k * b_k (or conj(a_k) * b_k)."""
    ya = unpack_spectrum(a)
    yb = unpack_spectrum(b)
    if conj_a:
        ya = np.conj(ya)
    return pack_spectrum(ya * yb)
