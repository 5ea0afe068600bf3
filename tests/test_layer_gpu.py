"""GPU tests of the autograd layer (BlockCirculantLinear) on the C ABI.

Gradients through torch.autograd are compared with the fp64 oracle (per row,
normwise relative error, the same gates as the kernel parity tests), and the
peak allocation of a forward + backward is checked to be exactly the layer's
outputs: no workspace.
"""

import pytest
import torch

import block_circulant_layers_amd as bcl
from block_circulant_layers_amd import synthetic as syn
from oracle import circulant_oracle as co
from tests.gpu_util import TOL, TORCH_DT, device_input, row_relerr, to_f64

pytestmark = pytest.mark.gpu


def _layer_with(c: torch.Tensor, weight_spectra: bool = False, deterministic: bool = False) -> bcl.BlockCirculantLinear:
    q, k, p = c.shape
    layer = bcl.BlockCirculantLinear(k * p, q * p, p, device="cuda:0", weight_spectra=weight_spectra,
                                     deterministic=deterministic)
    with torch.no_grad():
        layer.c.copy_(c)
    return layer


@pytest.mark.parametrize("weight_spectra", [False, True])
@pytest.mark.parametrize("batch,d_in,d_out,p,dtype,dense", [
    (3, 64, 64, 16, "f32", True),
    (5, 96, 160, 32, "bf16", True),
    (7, 1024, 512, 128, "f32", False),
    (4, 2048, 4096, 1024, "bf16", False),
    (6, 512, 256, 64, "f16", True),
])
def test_autograd_matches_oracle(batch, d_in, d_out, p, dtype, dense, weight_spectra):
    q, k = d_out // p, d_in // p
    print(f"layer autograd B={batch} d_in={d_in} d_out={d_out} p={p} {dtype} spectra={weight_spectra}", flush=True)
    x, xr = device_input((batch, d_in), syn.WL_TEST, syn.T_X, 11, dtype=dtype)
    c, cr = device_input((q, k, p), syn.WL_TEST, syn.T_C, 11, scale=1 / d_in**0.5)
    dy, dyr = device_input((batch, d_out), syn.WL_TEST, syn.T_DY, 11, dtype=dtype)
    layer = _layer_with(c, weight_spectra)
    x.requires_grad_(True)
    y = layer(x)
    y.backward(dy)
    torch.cuda.synchronize()
    if dense:
        yo = co.circulant_forward_dense(xr, cr)
        dxo, dco = co.circulant_backward_dense(xr, cr, dyr)
    else:
        yo = co.circulant_forward_fft(xr, cr)
        dxo, dco = co.circulant_backward_fft(xr, cr, dyr)
    assert y.dtype == TORCH_DT[dtype] and x.grad.dtype == TORCH_DT[dtype] and layer.c.grad.dtype == torch.float32
    assert row_relerr(to_f64(y), yo) <= TOL[dtype]
    assert row_relerr(to_f64(x.grad), dxo) <= TOL[dtype]
    assert row_relerr(to_f64(layer.c.grad).reshape(q * k, p), dco.reshape(q * k, p)) <= TOL["f32"]


def test_grad_accumulates_and_partial_needs():
    x, _ = device_input((4, 256), syn.WL_TEST, syn.T_X, 12)
    c, _ = device_input((2, 4, 64), syn.WL_TEST, syn.T_C, 12, scale=1 / 16)
    dy, _ = device_input((4, 128), syn.WL_TEST, syn.T_DY, 12)
    layer = _layer_with(c)
    layer(x).backward(dy)
    g1 = layer.c.grad.clone()
    layer(x).backward(dy)  # autograd adds the second dc into .grad
    torch.cuda.synchronize()
    assert torch.allclose(layer.c.grad, 2 * g1, rtol=1e-6, atol=1e-6)
    # x needs a gradient, c does not: the backward computes dx only
    layer.c.requires_grad_(False)
    x.requires_grad_(True)
    layer(x).backward(dy)
    dx_ref, _ = bcl.circulant_bwd(x.detach(), c, dy, need_dc=False)
    torch.cuda.synchronize()
    assert torch.equal(x.grad, dx_ref)


def test_second_backward_and_no_grad():
    # the forward's cleared gradient buffer serves one backward; a second
    # backward through the same graph (retain_graph) computes dc afresh, and
    # autograd adds it into .grad.  Under no_grad the forward clears nothing.
    x, xr = device_input((6, 512), syn.WL_TEST, syn.T_X, 14)
    c, cr = device_input((4, 4, 128), syn.WL_TEST, syn.T_C, 14, scale=1 / 512**0.5)
    dy, dyr = device_input((6, 512), syn.WL_TEST, syn.T_DY, 14)
    layer = _layer_with(c)
    y = layer(x)
    y.backward(dy, retain_graph=True)
    y.backward(dy)
    torch.cuda.synchronize()
    _, dco = co.circulant_backward_fft(xr, cr, dyr)
    assert row_relerr(to_f64(layer.c.grad).reshape(-1, 128), 2 * dco.reshape(-1, 128)) <= TOL["f32"]
    with torch.no_grad():
        y2 = layer(x)
    torch.cuda.synchronize()
    assert torch.equal(y2, y.detach())


def test_weight_spectra_steps_and_kept_spectra():
    # with weight_spectra: a frozen c (dx only) through circulant_fwd_step /
    # circulant_bwd_spec, two training steps adding into .grad, and forwards
    # without grad that reuse the kept spectra until c changes
    x, xr = device_input((6, 512), syn.WL_TEST, syn.T_X, 15, dtype="bf16")
    c, cr = device_input((4, 4, 128), syn.WL_TEST, syn.T_C, 15, scale=1 / 512**0.5)
    dy, dyr = device_input((6, 512), syn.WL_TEST, syn.T_DY, 15, dtype="bf16")
    layer = _layer_with(c, weight_spectra=True)
    layer(x).backward(dy)
    layer(x).backward(dy)
    torch.cuda.synchronize()
    _, dco = co.circulant_backward_fft(xr, cr, dyr)
    assert row_relerr(to_f64(layer.c.grad).reshape(-1, 128), 2 * dco.reshape(-1, 128)) <= TOL["f32"]
    layer.c.requires_grad_(False)
    xg = x.detach().clone().requires_grad_(True)
    layer(xg).backward(dy)
    dxo, _ = co.circulant_backward_fft(xr, cr, dyr)
    torch.cuda.synchronize()
    assert row_relerr(to_f64(xg.grad), dxo) <= TOL["bf16"]
    with torch.no_grad():
        y1 = layer(x)
        cs1 = layer._cs
        y2 = layer(x)
        assert layer._cs is cs1  # kept
        layer.c.mul_(2.0)  # c changes: the spectra are computed again
        y3 = layer(x)
        assert layer._cs is not cs1
    torch.cuda.synchronize()
    yo = co.circulant_forward_fft(xr, cr)
    assert torch.equal(y1, y2)
    assert row_relerr(to_f64(y1), yo) <= TOL["bf16"] and row_relerr(to_f64(y3), 2 * yo) <= TOL["bf16"]


@pytest.mark.parametrize("batch,d,p,dtype", [(256, 4096, 128, "bf16"), (2048, 4096, 1024, "bf16"), (33, 512, 16, "f32")])
def test_deterministic_layer(batch, d, p, dtype):
    # deterministic=True: c.grad is bitwise the same over five steps and
    # matches the oracle; x.grad (no token sum) is the default layer's bit for bit
    print(f"deterministic layer B={batch} D={d} p={p} {dtype}", flush=True)
    x, xr = device_input((batch, d), syn.WL_TEST, syn.T_X, 16, dtype=dtype)
    c, cr = device_input((d // p, d // p, p), syn.WL_TEST, syn.T_C, 16, scale=1 / d**0.5)
    dy, dyr = device_input((batch, d), syn.WL_TEST, syn.T_DY, 16, dtype=dtype)
    layer, ref = _layer_with(c, deterministic=True), _layer_with(c)
    runs = []
    for _ in range(5):
        layer.c.grad = None
        xg = x.detach().clone().requires_grad_(True)
        layer(xg).backward(dy)
        runs.append((layer.c.grad.clone(), xg.grad.clone()))
    xg = x.detach().clone().requires_grad_(True)
    ref(xg).backward(dy)
    torch.cuda.synchronize()
    for gc, gx in runs:
        assert torch.equal(gc, runs[0][0]) and torch.equal(gx, xg.grad)
    dxo, dco = co.circulant_backward_fft(xr, cr, dyr)
    assert row_relerr(to_f64(runs[0][0]).reshape(-1, p), dco.reshape(-1, p)) <= TOL["f32"]
    assert row_relerr(to_f64(runs[0][1]), dxo) <= TOL[dtype]


def test_token_axes_and_transposed_input():
    # activations shaped (sequences, tokens, features), the leading axes being
    # tokens alike, and a non-contiguous input (the layer makes it contiguous)
    p, d_in, d_out = 128, 512, 256
    q, k = d_out // p, d_in // p
    x, xr = device_input((3, 5, d_in), syn.WL_TEST, syn.T_X, 13, dtype="bf16")
    c, cr = device_input((q, k, p), syn.WL_TEST, syn.T_C, 13, scale=1 / d_in**0.5)
    dy, dyr = device_input((3, 5, d_out), syn.WL_TEST, syn.T_DY, 13, dtype="bf16")
    layer = _layer_with(c)
    xt = x.transpose(0, 1).detach().requires_grad_(True)  # (5, 3, d_in), not contiguous
    y = layer(xt)
    y.backward(dy.transpose(0, 1))
    torch.cuda.synchronize()
    assert y.shape == (5, 3, d_out)
    xo = xr.transpose(1, 0, 2).reshape(-1, d_in)
    dyo = dyr.transpose(1, 0, 2).reshape(-1, d_out)
    dxo, dco = co.circulant_backward_dense(xo, cr, dyo)
    assert row_relerr(to_f64(y).reshape(-1, d_out), co.circulant_forward_dense(xo, cr)) <= TOL["bf16"]
    assert row_relerr(to_f64(xt.grad).reshape(-1, d_in), dxo) <= TOL["bf16"]
    assert row_relerr(to_f64(layer.c.grad).reshape(q * k, p), dco.reshape(q * k, p)) <= TOL["f32"]


def _nbytes(t: torch.Tensor) -> int:
    # the caching allocator rounds every block up to 512 bytes
    return -(-t.numel() * t.element_size() // 512) * 512


@pytest.mark.parametrize("weight_spectra", [False, True])
@pytest.mark.parametrize("batch,d,p,dtype", [(256, 4096, 128, "bf16"), (256, 4096, 512, "bf16"),
                                             (256, 4096, 4096, "bf16"), (2048, 4096, 1024, "bf16"),
                                             (1, 4096, 128, "f32")])
def test_zero_workspace(batch, d, p, dtype, weight_spectra):
    """Peak allocation of forward + backward = y + dx + dc exactly (+ the
    weight spectra, the size of c, with weight_spectra)."""
    print(f"layer workspace B={batch} D={d} p={p} {dtype} spectra={weight_spectra}", flush=True)
    x, _ = device_input((batch, d), syn.WL_TEST, syn.T_X, 13, dtype=dtype)
    c, _ = device_input((d // p, d // p, p), syn.WL_TEST, syn.T_C, 13, scale=1 / d**0.5)
    dy, _ = device_input((batch, d), syn.WL_TEST, syn.T_DY, 13, dtype=dtype)
    layer = _layer_with(c, weight_spectra)
    x.requires_grad_(True)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    y = layer(x)
    y.backward(dy)
    torch.cuda.synchronize()
    peak = torch.cuda.max_memory_allocated() - before
    spectra = _nbytes(layer.c) if weight_spectra else 0
    assert peak == _nbytes(y) + _nbytes(x.grad) + _nbytes(layer.c.grad) + spectra, peak
