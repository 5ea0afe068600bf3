"""GPU parity of the layer calls that take the weights as packed spectra.

circulant_weight_spectra and circulant_fwd_step write cs = FFT(c) per weight
row (Paper-Notes page, "Squeeze" packing); circulant_fwd_spec and
circulant_bwd_spec compute the products of "循环矩阵训练适配" from cs.  Every
output is compared with the fp64 oracle per row (the gates of
test_circulant_gpu.py), cs with the oracle's packed forward of each row of c;
the two ways of writing cs agree bit for bit (the same transform of the same
rows).
"""

import pytest
import torch

import block_circulant_layers_amd as bcl
from block_circulant_layers_amd import synthetic as syn
from oracle import circulant_oracle as co
from oracle import rdfft_oracle as ro
from tests.gpu_util import TOL, device_input, row_relerr, to_f64

pytestmark = pytest.mark.gpu


def _say(*a):
    print(*a, flush=True)


def _inputs(batch, d_in, d_out, p, dtype, workload=syn.WL_TEST, index=0, c_scale=None):
    q, k = d_out // p, d_in // p
    x, xr = device_input((batch, d_in), workload, syn.T_X, index, dtype=dtype)
    c, cr = device_input((q, k, p), workload, syn.T_C, index, scale=c_scale or d_in**-0.5, dtype="f32")
    dy, dyr = device_input((batch, d_out), workload, syn.T_DY, index, dtype=dtype)
    return (x, c, dy), (xr, cr, dyr)


def _check_step(batch, d_in, d_out, p, dtype, want_dx=True, workload=syn.WL_TEST, index=0, c_scale=None):
    """circulant_fwd_step (y, cs, dc cleared from NaN), circulant_fwd_spec,
    circulant_bwd_spec overwriting dc, then adding into it."""
    (x, c, dy), (xr, cr, dyr) = _inputs(batch, d_in, d_out, p, dtype, workload, index, c_scale)
    _say(f"spectral weights B={batch} d_in={d_in} d_out={d_out} p={p} {dtype} dx={want_dx}")
    cs = torch.full_like(c, float("nan"))
    dc = torch.full_like(c, float("nan"))
    y = bcl.circulant_fwd_step(x, c, cs, dc=dc)
    cs2 = bcl.circulant_weight_spectra(c)
    y2 = bcl.circulant_fwd_spec(x, cs)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dc) == 0
    assert torch.equal(cs, cs2)
    ecs = row_relerr(to_f64(cs).reshape(-1, p), ro.rdfft_forward(cr.reshape(-1, p)))
    yo = co.circulant_forward_fft(xr, cr)
    ey, ey2 = row_relerr(to_f64(y), yo), row_relerr(to_f64(y2), yo)
    dx, _ = bcl.circulant_bwd_spec(x, cs, dy, dc=dc, need_dx=want_dx)
    torch.cuda.synchronize()
    dxo, dco = co.circulant_backward_fft(xr, cr, dyr)
    edc = row_relerr(to_f64(dc).reshape(-1, p), dco.reshape(-1, p))
    edx = row_relerr(to_f64(dx), dxo) if want_dx else 0.0
    dx2, _ = bcl.circulant_bwd_spec(x, cs, dy, dc=dc, need_dx=want_dx, accumulate=True)
    torch.cuda.synchronize()
    edc2 = row_relerr(to_f64(dc).reshape(-1, p), 2 * dco.reshape(-1, p))
    _say(f"  errors cs {ecs:.2e} y {ey:.2e} / {ey2:.2e} dx {edx:.2e} dc {edc:.2e} / {edc2:.2e}")
    assert ecs <= TOL["f32"] and ey <= TOL[dtype] and ey2 <= TOL[dtype] and edx <= TOL[dtype]
    assert edc <= TOL["f32"] and edc2 <= TOL["f32"]
    if want_dx:
        assert torch.equal(dx, dx2)
    return (x, c, dy, cs), (y, y2, dx)


@pytest.mark.parametrize("p", [2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096])
def test_weight_spectra_every_length(p):
    # 3 x 5 blocks, and 37 x 29 blocks for a ragged last round of rows
    for q, k in ((3, 5), (37, 29)):
        c, cr = device_input((q, k, p), syn.WL_TEST, syn.T_C, p + q, dtype="f32")
        cs = bcl.circulant_weight_spectra(c)
        torch.cuda.synchronize()
        err = row_relerr(to_f64(cs).reshape(-1, p), ro.rdfft_forward(cr.reshape(-1, p)))
        _say(f"weight spectra p={p} {q}x{k}: {err:.2e}")
        assert err <= TOL["f32"]
        assert torch.equal(c, torch.from_numpy(cr).float().to(c.device))  # c is read only


# small-p kernels (p < 64; p = 128 and 64 with more input blocks than one
# transform round holds), token-persistent tiles and the one-launch backward at
# every p, output tiles past the last block (q = 3, k = 5), a single token
SPEC_SHAPES = [
    (5, 8, 6, 2, "f32", True), (19, 48, 80, 16, "bf16", True), (9, 96, 64, 32, "f16", False),
    (9, 128, 320, 64, "bf16", True), (33, 640, 384, 128, "bf16", True), (33, 640, 384, 128, "f32", False),
    (3, 8192, 512, 128, "f32", True), (2, 8192, 256, 64, "bf16", True), (13, 512, 768, 256, "f16", True),
    (11, 1024, 512, 512, "bf16", True), (6, 2048, 4096, 1024, "f32", True), (5, 2048, 4096, 2048, "bf16", True),
    (3, 4096, 8192, 4096, "f32", True), (3, 8192, 4096, 4096, "bf16", False), (1, 4096, 4096, 4096, "bf16", True),
    (1, 512, 512, 64, "f32", True),
]


@pytest.mark.parametrize("batch,d_in,d_out,p,dtype,want_dx", SPEC_SHAPES)
def test_spec_parity_shapes(batch, d_in, d_out, p, dtype, want_dx):
    _check_step(batch, d_in, d_out, p, dtype, want_dx, index=p + d_in)


@pytest.mark.parametrize("p", [128, 512, 4096])
def test_spec_workload_d4096_b256(p):
    # single layer D = 4096, B = 256 tokens, bf16 activations, c ~ N(0, 1/D)
    _check_step(256, 4096, 4096, p, "bf16", workload=syn.WL_CIRC_LAYER, index=p, c_scale=1 / 64.0)


def test_spec_workload_adapter_shape():
    # one adapter of the 7B-decoder-shaped workload: 4096 x 4096, p = 1024, 2048 tokens
    _check_step(2048, 4096, 4096, 1024, "bf16", workload=syn.WL_CIRC_ADAPTERS, index=3, c_scale=1 / 64.0)


def test_spec_matches_time_domain_calls():
    # fp32 outputs of the two weight forms agree far inside the oracle gate
    (x, c, dy), _ = _inputs(256, 4096, 4096, 128, "f32", index=9)
    cs = bcl.circulant_weight_spectra(c)
    y, (dx, dc) = bcl.circulant_fwd_spec(x, cs), bcl.circulant_bwd_spec(x, cs, dy)
    y_ref, (dx_ref, dc_ref) = bcl.circulant_fwd(x, c), bcl.circulant_bwd(x, c, dy)
    torch.cuda.synchronize()
    assert row_relerr(to_f64(y), to_f64(y_ref)) <= 1e-6
    assert row_relerr(to_f64(dx), to_f64(dx_ref)) <= 1e-6
    assert row_relerr(to_f64(dc).reshape(-1, 128), to_f64(dc_ref).reshape(-1, 128)) <= 1e-6


def test_spec_empty_batch():
    c = torch.randn(2, 3, 16, device="cuda:0")
    x = torch.empty(0, 48, device="cuda:0")
    cs = torch.full_like(c, float("nan"))
    dc = torch.full_like(c, 5.0)
    y = bcl.circulant_fwd_step(x, c, cs, dc=dc)
    torch.cuda.synchronize()
    assert y.shape == (0, 32)
    assert torch.count_nonzero(dc) == 0
    assert torch.equal(cs, bcl.circulant_weight_spectra(c))
    dc.fill_(5.0)
    bcl.circulant_fwd_spec(x, cs, dc=dc)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dc) == 0
    dy = torch.empty(0, 32, device="cuda:0")
    dc.fill_(2.0)
    bcl.circulant_bwd_spec(x, cs, dy, dc=dc, need_dx=False, accumulate=True)
    torch.cuda.synchronize()
    assert torch.all(dc == 2.0)
    bcl.circulant_bwd_spec(x, cs, dy, dc=dc, need_dx=False)
    torch.cuda.synchronize()
    assert torch.count_nonzero(dc) == 0
