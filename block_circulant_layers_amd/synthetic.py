"""Seeded synthetic inputs shared by the tests, the smoke check and the benchmark.

This module holds no arithmetic of the method: it only draws numbers.  Both
the HIP path and the fp64 oracle are fed from here, so neither side ever
produces the other's inputs.

Every tensor is drawn as float64 standard normals from
``numpy.random.default_rng(SeedSequence([workload, tensor, index]))`` and
scaled; the caller casts it to the device dtype (bf16 by round-to-nearest-even
through torch) and hands the *cast* values to the oracle, so input rounding is
never charged to the kernel.
"""

from __future__ import annotations

import numpy as np

# workload ids (one per benchmark / test configuration)
WL_CIRC_SMALL = 0  # D=64, p=16, B=2 block-circulant layer
WL_RDFFT_512 = 1  # 4096 rows x 512
WL_RDFFT_LARGE = 2  # 4096 rows x 4096 and 16384 rows x 128
WL_CIRC_LAYER = 3  # D=4096, B=256, p in {128, 512, 4096}
WL_CIRC_ADAPTERS = 4  # 128 adapters 4096x4096, p=1024, 2048 tokens
WL_TEST = 99  # ad-hoc test shapes

# tensor ids
T_X = 0
T_C = 1
T_DY = 2


def normal(shape, workload: int, tensor: int, index: int = 0, scale: float = 1.0) -> np.ndarray:
    """float64 N(0, scale^2) array of ``shape`` from the seed (workload, tensor, index)."""
    rng = np.random.default_rng(np.random.SeedSequence([int(workload), int(tensor), int(index)]))
    return rng.standard_normal(shape) * scale


def cast_like_device(a: np.ndarray, dtype: str):
    """Round a float64 array to the device dtype ("f32", "bf16" or "f16").

    Returns (torch CPU tensor in that dtype, float64 numpy array of the rounded
    values).  16-bit rounding is torch's round-to-nearest-even.
    """
    import torch

    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float64))
    if dtype == "f32":
        tt = t.to(torch.float32)
    elif dtype == "bf16":
        tt = t.to(torch.bfloat16)
    elif dtype == "f16":
        tt = t.to(torch.float16)
    else:
        raise ValueError(f"unknown dtype {dtype!r}")
    return tt, tt.to(torch.float64).numpy()


def torch_normal(shape, workload: int, tensor: int, index: int = 0, scale: float = 1.0, dtype=None, device="cuda:0"):
    """N(0, scale^2) tensor drawn on `device` by torch's Philox generator seeded
    from (workload, tensor, index); used for the large benchmark buffers where
    drawing float64 on the host would dominate the run.  The oracle side of a
    comparison reads back the same device values."""
    import torch

    seed = int(np.random.SeedSequence([int(workload), int(tensor), int(index)]).generate_state(1, np.uint64)[0]) & (
        (1 << 63) - 1
    )
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(*shape, generator=g, device=device, dtype=torch.float32)
    if scale != 1.0:
        t.mul_(scale)
    return t if dtype is None else t.to(dtype)
