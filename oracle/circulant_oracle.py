"""fp64 oracle for block-circulant layers -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It shares no code with the HIP library.

The layer (Paper-Notes page, "循环矩阵训练适配"; scime.ai page, "Approach"):
a weight W of shape (D_out, D_in) is cut into q x k blocks of size p x p
(q = D_out / p, k = D_in / p).  Block (i, j) is the circulant matrix generated
by the vector c[i, j, :] of length p:

    W[i*p + a, j*p + b] = c[i, j, (a - b) mod p],

so that circ(c) x equals IFFT(FFT(c) * FFT(x)) (the pages' formula; this
first-column convention is the one that formula fixes).  For tokens x (rows
of length D_in):

    forward   y  = x W^T                       (y_i = sum_j C_ij x_j)
    backward  dx = dy W                        (dx_j = sum_i C_ij^T dy_i)
              dc[i, j, t] = sum_b sum_a dy[b, i*p+a] x[b, j*p + (a-t) mod p]

dc is the gradient of sum(dy * y) with respect to c: every entry of W that
holds c[i, j, t] contributes its dW.  There is no bias (the pages mention
none); dc is the sum over all tokens.

Two independent formulations:
  * ``*_dense``: the definition above, with the dense W materialised
    (small and medium shapes);
  * ``*_fft``: the pages' formula in the frequency domain, float64 complex
    FFT (numpy) as the DFT primitive:
        y_i  = IFFT( sum_j FFT(c_ij) * FFT(x_j) )
        dx_j = IFFT( sum_i conj(FFT(c_ij)) * FFT(dy_i) )
        dc_ij = IFFT( sum_b conj(FFT(x_bj)) * FFT(dy_bi) )
    (Paper-Notes page, section "循环矩阵训练适配": the gradients are products
    of packed spectra as well, so they stay conjugate-symmetric).
"""

from __future__ import annotations

import numpy as np

__all__ = [
    "block_circulant_weight",
    "circulant_forward_dense",
    "circulant_backward_dense",
    "circulant_forward_fft",
    "circulant_backward_fft",
]


def _shapes(x_cols: int, c: np.ndarray) -> tuple[int, int, int]:
    if c.ndim != 3:
        raise ValueError("c must have shape (q, k, p)")
    q, k, p = c.shape
    if k * p != x_cols:
        raise ValueError(f"x has {x_cols} columns, c implies D_in = {k * p}")
    return q, k, p


def block_circulant_weight(c: np.ndarray) -> np.ndarray:
    """Dense W (q*p, k*p) with W[i*p+a, j*p+b] = c[i, j, (a-b) mod p]."""
    c = np.asarray(c, dtype=np.float64)
    q, k, p = c.shape
    a = np.arange(p)[:, None]
    b = np.arange(p)[None, :]
    idx = (a - b) % p  # (p, p)
    blocks = c[:, :, idx]  # (q, k, p, p): blocks[i, j, a, b]
    return blocks.transpose(0, 2, 1, 3).reshape(q * p, k * p)


def circulant_forward_dense(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    _shapes(x.shape[-1], c)
    return x @ block_circulant_weight(c).T


def circulant_backward_dense(x: np.ndarray, c: np.ndarray, dy: np.ndarray):
    """Returns (dx, dc) from the dense definition."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    q, k, p = _shapes(x.shape[-1], c)
    w = block_circulant_weight(c)
    dx = dy @ w
    dw = dy.T @ x  # (q*p, k*p), dW[i*p+a, j*p+b'] = sum_b dy[b, i*p+a] x[b, j*p+b']
    dwb = dw.reshape(q, p, k, p).transpose(0, 2, 1, 3)  # (q, k, a, b')
    dc = np.zeros((q, k, p), dtype=np.float64)
    a = np.arange(p)
    for t in range(p):
        # entries with (a - b') mod p == t, i.e. b' = (a - t) mod p
        dc[:, :, t] = dwb[:, :, a, (a - t) % p].sum(axis=-1)
    return dx, dc


def circulant_forward_fft(x: np.ndarray, c: np.ndarray) -> np.ndarray:
    x = np.asarray(x, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    q, k, p = _shapes(x.shape[-1], c)
    xf = np.fft.fft(x.reshape(x.shape[0], k, p), axis=-1)  # (B, k, p)
    cf = np.fft.fft(c, axis=-1)  # (q, k, p)
    yf = np.einsum("ijf,bjf->bif", cf, xf)
    return np.fft.ifft(yf, axis=-1).real.reshape(x.shape[0], q * p)


def circulant_backward_fft(x: np.ndarray, c: np.ndarray, dy: np.ndarray):
    """Returns (dx, dc) from the pages' frequency-domain formulas."""
    x = np.asarray(x, dtype=np.float64)
    dy = np.asarray(dy, dtype=np.float64)
    c = np.asarray(c, dtype=np.float64)
    q, k, p = _shapes(x.shape[-1], c)
    nb = x.shape[0]
    xf = np.fft.fft(x.reshape(nb, k, p), axis=-1)  # (B, k, p)
    gf = np.fft.fft(dy.reshape(nb, q, p), axis=-1)  # (B, q, p)
    cf = np.fft.fft(c, axis=-1)
    dxf = np.einsum("ijf,bif->bjf", np.conj(cf), gf)
    dcf = np.einsum("bjf,bif->ijf", np.conj(xf), gf)
    dx = np.fft.ifft(dxf, axis=-1).real.reshape(nb, k * p)
    dc = np.fft.ifft(dcf, axis=-1).real
    return dx, dc
