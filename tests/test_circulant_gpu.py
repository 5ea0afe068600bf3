"""GPU parity of the block-circulant layer forward / backward against the fp64 oracle.

Outputs are compared per row (a token row of y or dx, a (i, j) row of dc):
normwise relative error, max over rows, <= 1e-5 for fp32-stored outputs,
<= 2e-2 for bf16-stored and <= 1e-3 for fp16-stored outputs (dc is always fp32).
"""

import numpy as np
import pytest
import torch

import block_circulant_layers_amd as bcl
from block_circulant_layers_amd import synthetic as syn
from oracle import circulant_oracle as co
from tests.gpu_util import TOL, device_input, row_relerr, to_f64

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _run(batch, d_in, d_out, p, dtype, workload=syn.WL_TEST, index=0, c_scale=1.0, dense=True):
    q, k = d_out // p, d_in // p
    x, xr = device_input((batch, d_in), workload, syn.T_X, index, dtype=dtype)
    c, cr = device_input((q, k, p), workload, syn.T_C, index, scale=c_scale, dtype="f32")
    dy, dyr = device_input((batch, d_out), workload, syn.T_DY, index, dtype=dtype)
    _say(f"circulant fwd/bwd B={batch} d_in={d_in} d_out={d_out} p={p} dtype={dtype}")
    y = bcl.circulant_fwd(x, c)
    dx, dc = bcl.circulant_bwd(x, c, dy)
    torch.cuda.synchronize()
    if dense:
        yo = co.circulant_forward_dense(xr, cr)
        dxo, dco = co.circulant_backward_dense(xr, cr, dyr)
    else:
        yo = co.circulant_forward_fft(xr, cr)
        dxo, dco = co.circulant_backward_fft(xr, cr, dyr)
    ey = row_relerr(to_f64(y), yo)
    edx = row_relerr(to_f64(dx), dxo)
    edc = row_relerr(to_f64(dc).reshape(q * k, p), dco.reshape(q * k, p))
    _say(f"  errors y {ey:.2e} dx {edx:.2e} dc {edc:.2e}")
    assert ey <= TOL[dtype] and edx <= TOL[dtype] and edc <= TOL["f32"], (ey, edx, edc)
    return (x, c, dy, y, dx, dc), (xr, cr, dyr)


def test_workload_d64_p16_b2():
    # D = 64, p = 16 (4 x 4 blocks), B = 2, fp32; dense-matrix oracle
    _run(2, 64, 64, 16, "f32", syn.WL_CIRC_SMALL)


SHAPES = [
    (5, 8, 6, 2), (3, 16, 8, 4), (7, 24, 40, 8), (19, 48, 80, 16), (9, 96, 64, 32), (9, 128, 320, 64),
    (33, 384, 256, 128), (13, 512, 768, 256), (11, 1024, 512, 512), (6, 2048, 4096, 1024),
    (5, 2048, 4096, 2048), (3, 4096, 8192, 4096), (3, 8192, 4096, 4096),
    # input-block counts past one transform round of the token-persistent kernel
    # (the fallback kernels run that direction): p = 64 with 128 input blocks,
    # p = 128 with 64, p = 1024 with 8
    (2, 8192, 256, 64), (3, 8192, 512, 128), (2, 8192, 2048, 1024),
    # a single token
    (1, 512, 512, 64), (1, 1024, 2048, 512), (1, 4096, 4096, 4096),
]


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("batch,d_in,d_out,p", SHAPES)
def test_parity_shapes(batch, d_in, d_out, p, dtype):
    _run(batch, d_in, d_out, p, dtype, index=p + d_in, dense=(d_in * d_out <= 4096 * 4096))


@pytest.mark.parametrize("p", [128, 512, 4096])
def test_workload_d4096_b256(p):
    # single layer D = 4096, B = 256 tokens, bf16 activations, fp32 c ~ N(0, 1/D)
    _run(256, 4096, 4096, p, "bf16", syn.WL_CIRC_LAYER, index=p, c_scale=1 / 64.0, dense=False)


@pytest.mark.parametrize("adapter", [0, 77])
def test_workload_adapter_shape(adapter):
    # one of the 128 adapters of the 7B-decoder-shaped workload, at its full shape:
    # 4096 x 4096, p = 1024 (4 x 4 blocks), 2048 tokens, bf16
    (x, c, dy, y, dx, dc), _ = _run(2048, 4096, 4096, 1024, "bf16", syn.WL_CIRC_ADAPTERS, index=adapter,
                                    c_scale=1 / 64.0, dense=False)


def test_adjoint_identities_on_gpu_outputs():
    (x, c, dy, y, dx, dc), _ = _run(512, 4096, 4096, 1024, "f32", index=5, c_scale=1 / 64.0, dense=False)
    s1 = float((dy.double() * y.double()).sum())
    s2 = float((dx.double() * x.double()).sum())
    s3 = float((dc.double() * c.double()).sum())
    assert abs(s1 - s2) <= 1e-5 * abs(s1) and abs(s1 - s3) <= 1e-5 * abs(s1)


def test_dc_overwritten_and_optional_outputs():
    batch, d, p = 40, 256, 64
    x, xr = device_input((batch, d), syn.WL_TEST, syn.T_X, 1)
    c, cr = device_input((d // p, d // p, p), syn.WL_TEST, syn.T_C, 1)
    dy, dyr = device_input((batch, d), syn.WL_TEST, syn.T_DY, 1)
    dxo, dco = co.circulant_backward_dense(xr, cr, dyr)
    dc = torch.full_like(c, float("nan"))
    dx = torch.full_like(x, float("nan"))
    bcl.circulant_bwd(x, c, dy, dx=dx, dc=dc)
    torch.cuda.synchronize()
    assert row_relerr(to_f64(dx), dxo) <= 1e-5
    assert row_relerr(to_f64(dc).reshape(-1, p), dco.reshape(-1, p)) <= 1e-5
    _, dc2 = bcl.circulant_bwd(x, c, dy, need_dx=False)
    dx2, none = bcl.circulant_bwd(x, c, dy, need_dc=False)
    torch.cuda.synchronize()
    assert none is None
    assert row_relerr(to_f64(dc2).reshape(-1, p), dco.reshape(-1, p)) <= 1e-5
    assert row_relerr(to_f64(dx2), dxo) <= 1e-5


@pytest.mark.parametrize("batch,d,p,dtype", [(256, 4096, 128, "bf16"), (96, 2048, 512, "f32"), (512, 4096, 1024, "bf16"),
                                            (40, 4096, 2048, "f16"), (64, 4096, 4096, "f32"), (70, 1024, 64, "bf16"),
                                            (45, 2048, 256, "f32")])
def test_backward_single_outputs(batch, d, p, dtype):
    # dx alone and dc alone take other launches than the two together (one
    # launch holds both where the row length allows; dc alone adds packed
    # spectra and transforms dc back afterwards at p <= 128, time-domain sums
    # from p = 256): each against the oracle
    q = k = d // p
    x, xr = device_input((batch, d), syn.WL_TEST, syn.T_X, p + 3, dtype=dtype)
    c, cr = device_input((q, k, p), syn.WL_TEST, syn.T_C, p + 3, scale=1 / np.sqrt(d), dtype="f32")
    dy, dyr = device_input((batch, d), syn.WL_TEST, syn.T_DY, p + 3, dtype=dtype)
    _say(f"circulant bwd single outputs B={batch} D={d} p={p} dtype={dtype}")
    dxo, dco = co.circulant_backward_fft(xr, cr, dyr)
    dx_both, dc_both = bcl.circulant_bwd(x, c, dy)
    _, dc_only = bcl.circulant_bwd(x, c, dy, need_dx=False)
    dx_only, _ = bcl.circulant_bwd(x, c, dy, need_dc=False)
    torch.cuda.synchronize()
    for dx in (dx_both, dx_only):
        assert row_relerr(to_f64(dx), dxo) <= TOL[dtype]
    for dc in (dc_both, dc_only):
        assert row_relerr(to_f64(dc).reshape(-1, p), dco.reshape(-1, p)) <= TOL["f32"]
    # the dx products are the same arithmetic in either launch
    assert torch.equal(dx_both, dx_only)


def test_empty_batch():
    c = torch.randn(2, 2, 16, device="cuda:0")
    x = torch.empty(0, 32, device="cuda:0")
    y = bcl.circulant_fwd(x, c)
    dc = torch.full_like(c, 5.0)
    bcl.circulant_bwd(x, c, torch.empty(0, 32, device="cuda:0"), dc=dc)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)
    assert torch.count_nonzero(dc) == 0  # sum over no tokens


def test_identity_and_shift_weights():
    p, d, batch = 256, 1024, 8
    x, xr = device_input((batch, d), syn.WL_TEST, syn.T_X, 9)
    c = torch.zeros(d // p, d // p, p, device="cuda:0")
    for i in range(d // p):
        c[i, i, 0] = 1.0  # W = I
    y = bcl.circulant_fwd(x, c)
    c2 = torch.zeros(1, 1, p, device="cuda:0")
    c2[0, 0, 3] = 1.0  # cyclic shift by 3
    x1 = x[:, :p].contiguous()
    y2 = bcl.circulant_fwd(x1, c2)
    torch.cuda.synchronize()
    assert np.allclose(to_f64(y), xr, atol=1e-5)
    assert np.allclose(to_f64(y2), np.roll(xr[:, :p], 3, axis=1), atol=1e-5)
