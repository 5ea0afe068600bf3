"""GPU tests of the packed <-> complex-bin utilities (rdfft_unpack / rdfft_pack).

They only move values (widening 16-bit storage, or rounding to it once), so
parity with the oracle's pack/unpack of the packed layout is bit-exact.  The
complex view of a forward transform is also checked against the oracle's
DFT bins directly.
"""

import numpy as np
import pytest
import torch

import block_circulant_layers_amd as bcl
from block_circulant_layers_amd import synthetic as syn
from oracle import rdfft_oracle as ro
from tests.gpu_util import TOL, TORCH_DT, device_input, row_relerr, to_f64

pytestmark = pytest.mark.gpu

P_LIST = [2, 4, 16, 128, 512, 4096]


def _bins(z: np.ndarray) -> np.ndarray:
    """oracle: packed rows -> (rows, p/2 + 1, 2) float64 (Re, Im) of bins 0..p/2"""
    y = ro.unpack_spectrum(z)[..., : z.shape[-1] // 2 + 1]
    return np.stack([y.real, y.imag], axis=-1)


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("p", P_LIST)
def test_unpack_exact(p, dtype):
    rows = 3 + 8192 // p
    print(f"unpack rows={rows} p={p} {dtype}", flush=True)
    z, zr = device_input((rows, p), syn.WL_TEST, syn.T_X, 200 + p, dtype=dtype)
    spec = bcl.rdfft_unpack(z)
    torch.cuda.synchronize()
    assert spec.shape == (rows, p // 2 + 1, 2)
    assert np.array_equal(to_f64(spec), _bins(zr))


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("p", P_LIST)
def test_pack_exact(p, dtype):
    rows = 3 + 8192 // p
    print(f"pack rows={rows} p={p} {dtype}", flush=True)
    s, sr = device_input((rows, p // 2 + 1, 2), syn.WL_TEST, syn.T_C, 300 + p)
    packed = torch.empty(rows, p, dtype=TORCH_DT[dtype], device="cuda:0")
    bcl.rdfft_pack(s, packed)
    torch.cuda.synchronize()
    # oracle: the complex bins (Im of bins 0 and p/2 dropped: a real row has them zero)
    y = sr[..., 0] + 1j * sr[..., 1]
    y[:, 0] = y[:, 0].real
    y[:, -1] = y[:, -1].real
    full = np.concatenate([y, np.conj(y[:, -2:0:-1])], axis=1)
    want, _ = syn.cast_like_device(ro.pack_spectrum(full), dtype)
    assert torch.equal(packed.cpu(), want)


@pytest.mark.parametrize("p", P_LIST)
def test_roundtrips(p):
    z, _ = device_input((7, p), syn.WL_TEST, syn.T_X, 400 + p)
    back = torch.empty_like(z)
    bcl.rdfft_pack(bcl.rdfft_unpack(z), back)
    torch.cuda.synchronize()
    assert torch.equal(back, z)


@pytest.mark.parametrize("p", [8, 512, 4096])
def test_forward_then_unpack_is_the_dft(p):
    x, xr = device_input((5, p), syn.WL_TEST, syn.T_X, 500 + p)
    spec = bcl.rdfft_unpack(bcl.rdfft_forward(x))
    torch.cuda.synchronize()
    want = np.fft.rfft(xr, axis=-1)
    got = to_f64(spec)
    err = row_relerr(np.concatenate([got[..., 0], got[..., 1]], -1), np.concatenate([want.real, want.imag], -1))
    assert err <= TOL["f32"], err


def test_empty_and_no_allocation():
    z = torch.empty(0, 512, device="cuda:0")
    spec = torch.empty(0, 257, 2, device="cuda:0")
    bcl.rdfft_unpack(z, spec)
    bcl.rdfft_pack(spec, z)
    z, _ = device_input((64, 512), syn.WL_TEST, syn.T_X, 600)
    spec = torch.empty(64, 257, 2, device="cuda:0")
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    bcl.rdfft_unpack(z, spec)
    bcl.rdfft_pack(spec, z)
    torch.cuda.synchronize()
    assert torch.cuda.max_memory_allocated() == before
