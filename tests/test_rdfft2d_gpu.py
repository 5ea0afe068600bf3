"""GPU parity of the 2D packed real FFT (rdfft2d_forward / rdfft2d_inverse)
against the fp64 oracle (oracle/rdfft2d_oracle.py).

Error metric: ||gpu - oracle||_2 / ||oracle||_2 of every row and of every
column of every array, the maximum of all of them (a single wrong column or
row of a large array fails the gate, which a norm over the whole array would
dilute).  Gates: 1e-5 for fp32; 16-bit storage is rounded after each of the three
passes, so the gates are three roundings: bf16 3 x 2^-9 = 5.9e-3 (gate 2e-2,
as for 1D) and fp16 3 x 2^-11 = 1.5e-3 (gate 3e-3).
"""

import numpy as np
import pytest
import torch

import block_circulant_layers_amd as bcl
from block_circulant_layers_amd import synthetic as syn
from oracle import rdfft2d_oracle as r2
from tests.gpu_util import device_input, row_relerr, to_f64

pytestmark = pytest.mark.gpu

TOL2D = {"f32": 1e-5, "bf16": 2e-2, "f16": 3e-3}
SHAPES = [(3, 2, 8), (2, 8, 2), (2, 4, 4), (2, 16, 32), (2, 64, 512), (1, 1024, 1024), (1, 4096, 64),
          (2, 128, 8192), (1, 32, 32768), (2, 4096, 16), (3, 2048, 32)]


def rowcol_relerr(got, want):
    """Largest normwise relative error over every row and every column of
    every [h, w] array of got/want [n, h, w]."""
    return max(row_relerr(got, want), row_relerr(np.swapaxes(got, -1, -2), np.swapaxes(want, -1, -2)))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("n,h,w", SHAPES)
def test_parity(n, h, w, dtype):
    print(f"rdfft2d n={n} h={h} w={w} {dtype}", flush=True)
    x, xr = device_input((n, h, w), syn.WL_TEST, syn.T_X, 700 + h + w, dtype=dtype)
    bcl.rdfft2d_forward(x)
    torch.cuda.synchronize()
    z = to_f64(x)
    ef = rowcol_relerr(z, r2.rdfft2d_forward(xr))
    bcl.rdfft2d_inverse(x)
    torch.cuda.synchronize()
    ei = rowcol_relerr(to_f64(x), r2.rdfft2d_inverse(z))
    print(f"  errors fwd {ef:.2e} inv {ei:.2e}", flush=True)
    assert ef <= TOL2D[dtype] and ei <= TOL2D[dtype], (ef, ei)


def test_full_size_4096x4096():
    # the benchmarked array, in the launch configuration the benchmark times
    print("rdfft2d n=1 h=4096 w=4096 f32", flush=True)
    x, xr = device_input((1, 4096, 4096), syn.WL_TEST, syn.T_X, 4242)
    bcl.rdfft2d_forward(x)
    torch.cuda.synchronize()
    z = to_f64(x)
    assert rowcol_relerr(z, r2.rdfft2d_forward(xr)) <= TOL2D["f32"]
    bcl.rdfft2d_inverse(x)
    torch.cuda.synchronize()
    assert rowcol_relerr(to_f64(x), r2.rdfft2d_inverse(z)) <= TOL2D["f32"]


@pytest.mark.parametrize("h,w", [(16, 16), (256, 128)])
def test_inverse_accepts_any_array_and_roundtrip(h, w):
    z, zr = device_input((2, h, w), syn.WL_TEST, syn.T_DY, h * w)
    bcl.rdfft2d_inverse(z)
    torch.cuda.synchronize()
    assert rowcol_relerr(to_f64(z), r2.rdfft2d_inverse(zr)) <= 1e-5
    bcl.rdfft2d_forward(z)
    torch.cuda.synchronize()
    assert rowcol_relerr(to_f64(z), zr) <= 1e-5


def test_closed_form_delta_and_empty():
    x = torch.zeros(1, 8, 16, device="cuda:0")
    x[0, 0, 0] = 1.0
    bcl.rdfft2d_forward(x)
    torch.cuda.synchronize()
    want = np.zeros((8, 16))
    want[:5, 0] = want[:5, 8] = 1.0
    want[:, 1:8] = 1.0
    assert np.allclose(to_f64(x)[0], want, atol=1e-6)
    e = torch.empty(0, 8, 16, device="cuda:0")
    bcl.rdfft2d_forward(e)
    bcl.rdfft2d_inverse(e)
    torch.cuda.synchronize()


def test_no_device_allocation():
    x, _ = device_input((1, 1024, 1024), syn.WL_TEST, syn.T_X, 9)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    bcl.rdfft2d_forward(x)
    bcl.rdfft2d_inverse(x)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == before
