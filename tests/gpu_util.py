"""Helpers shared by the GPU parity tests (input preparation and error metric only)."""

from __future__ import annotations

import numpy as np
import torch

from block_circulant_layers_amd import synthetic as syn

# gates of the parity tests: normwise relative error, max over rows
# fp16 storage: one rounding of the output at unit roundoff 2^-11 bounds the
# normwise error by 4.9e-4 (inputs are rounded before the oracle sees them and
# fp32 arithmetic adds ~1e-6), so 1e-3 leaves a factor of two
TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 1e-3}
TORCH_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def device_input(shape, workload, tensor, index=0, scale=1.0, dtype="f32"):
    """Seeded N(0, scale^2) input on cuda:0 in `dtype` plus the float64 copy of
    exactly the values the GPU sees (the oracle's input)."""
    a = syn.normal(shape, workload, tensor, index, scale)
    t, ref = syn.cast_like_device(a, dtype)
    return t.to("cuda:0"), ref


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().to("cpu", torch.float64).numpy()


def row_relerr(got: np.ndarray, want: np.ndarray) -> float:
    """max over rows of ||got - want||_2 / ||want||_2 (rows = last axis)."""
    got = got.reshape(-1, got.shape[-1])
    want = want.reshape(-1, want.shape[-1])
    num = np.sqrt(np.sum((got - want) ** 2, axis=1))
    den = np.sqrt(np.sum(want**2, axis=1))
    den = np.where(den == 0, 1.0, den)
    return float(np.max(num / den)) if len(num) else 0.0
