"""Autograd function and module of the block-circulant layer on the C ABI.

The layer computes, for every token row x (d_in = k p features) and
parameters c of shape (q, k, p), y_i = sum_j IFFT(FFT(c_ij) * FFT(x_j)): block
(i, j) is the circulant matrix whose first column is c_ij, applied to input
chunk j and summed into output chunk i (Paper-Notes, "循环矩阵训练适配": the
circulant product through the in-place transform and its use in training).
Forward and backward run in the library's fused kernels; nothing here
computes, and there is no CPU path.  When c needs a gradient, the forward
(``circulant_fwd_zero``) also clears a buffer for it in the same launch and the
backward (``circulant_bwd_acc``) adds the token sum into that buffer, so a
step takes two launches and no separate clearing pass.  The backward
recomputes FFT(x) from the saved input rather than saving spectra, so a layer
keeps only what a dense Linear would keep (x, its parameters and, between the
passes, the parameter-sized gradient buffer).

With ``weight_spectra=True`` the layer also keeps the packed spectra of its
weight rows, one more parameter-sized buffer: a training step's forward
(``circulant_fwd_step``) writes them as it transforms the weights, and the
backward (``circulant_bwd_spec``) reads them instead of transforming the
weights again; without grad, the spectra are kept across calls until c
changes, and the forward (``circulant_fwd_spec``) transforms no weight rows.

With ``deterministic=True`` the backward computes dc with ``circulant_bwd_det``:
each token range's partial sums go to a workspace (allocated through torch,
one q k p slice per range) and are summed in a fixed order, so c's gradient
is bitwise the same from run to run.
"""

from __future__ import annotations

import math

import torch

from .binding import (
    circulant_bwd,
    circulant_bwd_acc,
    circulant_bwd_det,
    circulant_bwd_spec,
    circulant_fwd,
    circulant_fwd_spec,
    circulant_fwd_step,
    circulant_fwd_zero,
    circulant_weight_spectra,
)

__all__ = ["BlockCirculantFunction", "BlockCirculantLinear"]


class BlockCirculantFunction(torch.autograd.Function):
    """y = block-circulant(c) x per token; gradients dx and dc from one backward call.

    ``grad_buffer``: the caller will need dc (grad mode on and c requires it),
    so the forward clears a gradient buffer in its launch.  Grad mode is off
    inside ``forward``, hence the caller decides.  ``spectra``: the forward
    also writes the weight spectra, which the backward reads.
    ``deterministic``: dc from ``circulant_bwd_det`` (no gradient buffer, no
    spectra).
    """

    @staticmethod
    def forward(ctx, x: torch.Tensor, c: torch.Tensor, grad_buffer: bool = False,
                spectra: bool = False, deterministic: bool = False) -> torch.Tensor:
        x = x.contiguous()
        c = c.contiguous()
        ctx.save_for_backward(x, c)
        ctx.dc = None
        ctx.cs = None
        ctx.det = deterministic
        if deterministic:
            return circulant_fwd(x, c)
        want_dc = grad_buffer and ctx.needs_input_grad[1]
        if want_dc:
            ctx.dc = torch.empty_like(c)  # cleared by the forward launch, filled by the backward
        if spectra and (ctx.needs_input_grad[0] or want_dc):
            ctx.cs = torch.empty_like(c)  # written by the forward launch, read by the backward
            return circulant_fwd_step(x, c, ctx.cs, dc=ctx.dc)
        if want_dc:
            return circulant_fwd_zero(x, c, ctx.dc)
        return circulant_fwd(x, c)

    @staticmethod
    def backward(ctx, dy: torch.Tensor):
        x, c = ctx.saved_tensors
        need_dx, need_dc = ctx.needs_input_grad[0], ctx.needs_input_grad[1]
        if not (need_dx or need_dc):
            return None, None, None, None, None
        dc, ctx.dc = ctx.dc, None  # zeroed buffer: good for one backward only
        dy = dy.contiguous()
        if ctx.det and need_dc:
            dx, dc = circulant_bwd_det(x, c, dy, need_dx=need_dx)
        elif ctx.cs is not None:
            if need_dc and dc is not None:
                dx, dc = circulant_bwd_spec(x, ctx.cs, dy, dc=dc, need_dx=need_dx, accumulate=True)
            else:
                dx, dc = circulant_bwd_spec(x, ctx.cs, dy, need_dx=need_dx, need_dc=need_dc)
        elif need_dc and dc is not None:
            dx, dc = circulant_bwd_acc(x, c, dy, dc, need_dx=need_dx)
        else:  # dx alone has no token sum, so it is the same in every mode
            dx, dc = circulant_bwd(x, c, dy, need_dx=need_dx, need_dc=need_dc)
        return dx, dc, None, None, None


class BlockCirculantLinear(torch.nn.Module):
    """A d_in -> d_out layer whose weight is a (d_out/p) x (d_in/p) grid of
    p x p circulant blocks, stored as their first columns c (fp32, q x k x p).

    Activations may be float32 or bfloat16 and must live on a GPU.  ``c`` is
    initialised N(0, 1/d_in), the variance that keeps y at the scale of x.
    ``weight_spectra``: keep the packed spectra of the weight rows in one more
    buffer of c's size; ``deterministic``: a bitwise reproducible gradient of c
    (see the module docstring; the two do not combine).
    """

    def __init__(self, d_in: int, d_out: int, p: int, device=None, generator: torch.Generator | None = None,
                 weight_spectra: bool = False, deterministic: bool = False):
        super().__init__()
        if p < 2 or p & (p - 1) or d_in % p or d_out % p:
            raise ValueError("p must be a power of two >= 2 dividing d_in and d_out")
        if weight_spectra and deterministic:
            raise ValueError("weight_spectra and deterministic do not combine")
        self.d_in, self.d_out, self.p = d_in, d_out, p
        self.weight_spectra = weight_spectra
        self.deterministic = deterministic
        c = torch.empty(d_out // p, d_in // p, p, dtype=torch.float32, device=device)
        with torch.no_grad():
            c.normal_(0.0, 1.0 / math.sqrt(d_in), generator=generator)
        self.c = torch.nn.Parameter(c)
        self._cs = None  # spectra of c kept across calls without grad
        self._cs_of = None  # (data pointer, version) of the c they were computed from

    def forward(self, x: torch.Tensor) -> torch.Tensor:
        grad = torch.is_grad_enabled() and (self.c.requires_grad or x.requires_grad)
        if self.weight_spectra and not grad:
            key = (self.c.data_ptr(), self.c._version)
            if self._cs is None or self._cs_of != key or self._cs.device != self.c.device:
                self._cs = circulant_weight_spectra(self.c.detach())
                self._cs_of = key
            return circulant_fwd_spec(x.contiguous(), self._cs)
        self._cs = None
        return BlockCirculantFunction.apply(x, self.c, torch.is_grad_enabled() and self.c.requires_grad,
                                            self.weight_spectra, self.deterministic)

    def extra_repr(self) -> str:
        return (f"d_in={self.d_in}, d_out={self.d_out}, p={self.p}, weight_spectra={self.weight_spectra}, "
                f"deterministic={self.deterministic}")
