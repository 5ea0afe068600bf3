"""Autograd function and module of the block-circulant layer on the C ABI.

The layer computes, for every token row x (d_in = k p features) and
parameters c of shape (q, k, p), y_i = sum_j IFFT(FFT(c_ij) * FFT(x_j)): block
(i, j) is the circulant matrix whose first column is c_ij, applied to input
chunk j and summed into output chunk i (Paper-Notes, "循环矩阵训练适配": the
circulant product through the in-place transform and its use in training).
Forward and backward run in the library's fused kernels (``circulant_fwd`` and
``circulant_bwd``); nothing here computes, and there is no CPU path.  The
backward recomputes FFT(x) from the saved input rather than saving spectra,
so a layer keeps only what a dense Linear would keep (x and its parameters).
"""

from __future__ import annotations

import math

import torch

from .binding import circulant_bwd, circulant_fwd

__all__ = ["BlockCirculantFunction", "BlockCirculantLinear"]


class BlockCirculantFunction(torch.autograd.Function):
    """y = block-circulant(c) x per token; gradients dx and dc from one backward call."""

    @staticmethod
    def forward(ctx, x: torch.Tensor, c: torch.Tensor) -> torch.Tensor:
        x = x.contiguous()
        c = c.contiguous()
        ctx.save_for_backward(x, c)
        return circulant_fwd(x, c)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x, c = ctx.saved_tensors
        need_dx, need_dc = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_dx or need_dc):
            return None, None
        dx, dc = circulant_bwd(x, c, dy.contiguous(), need_dx=need_dx, need_dc=need_dc)
        return dx, dc


class BlockCirculantLinear(torch.nn.Module):
    """A d_in -> d_out layer whose weight is a (d_out/p) x (d_in/p) grid of
    p x p circulant blocks, stored as their first columns c (fp32, q x k x p).

    Activations may be float32 or bfloat16 and must live on a GPU.  ``c`` is
    initialised N(0, 1/d_in), the variance that keeps y at the scale of x.
    """

    def __init__(self, d_in: int, d_out: int, p: int, device=None, generator: torch.Generator | None = None):
        super().__init__()
        if p < 2 or p & (p - 1) or d_in % p or d_out % p:
            raise ValueError("p must be a power of two >= 2 dividing d_in and d_out")
        self.d_in, self.d_out, self.p = d_in, d_out, p
        c = torch.empty(d_out // p, d_in // p, p, dtype=torch.float32, device=device)
        with torch.no_grad():
            c.normal_(0.0, 1.0 / math.sqrt(d_in), generator=generator)
        self.c = torch.nn.Parameter(c)

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        return BlockCirculantFunction.apply(x, self.c)

    def extra_repr(self) -> str:
        return f"d_in={self.d_in}, d_out={self.d_out}, p={self.p}"
