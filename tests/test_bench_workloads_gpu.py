"""The circulant workloads in the launch configuration bench.py times.

bench.py's own setup functions build the inputs (bf16 token batches and
gradients drawn on the device, fp32 c) and the step closures; the steps are
captured in a HIP graph and replayed as the bench replays them, then checked
against the fp64 oracle (Paper-Notes, "循环矩阵训练适配"), which reads back the
device's input values:

- the single layer D=4096, B=256 at p = 128, 512 and 4096: one replayed
  rotation of 32 training steps; steps 0 and 31 in full (y and dx per token
  row, dc of step 31, which the rotation leaves in the buffer);
- the 128 adapters (4096x4096, p=1024, 2048 tokens): one replayed step;
  adapters 0, 64 and 127 in full;
each in both forms bench.py times: the weights transformed at every call, and
their spectra kept from forward to backward (circulant_fwd_step and
circulant_bwd_spec).

Every step of the rotation and every adapter is also checked through the
adjoint identities <dy, y> = <dx, x> (= <dc, c> where dc is at hand), which
hold for the exact linear map at any size.  y and dx are stored in bf16, so
their inner products carry the outputs' rounding; the gate is 2e-2 of the
products' natural scale rms(a) rms(b) sqrt(n), about 20 times the rounding's
spread, far below the error of a wrong or missing launch.
"""

import math

import pytest
import torch

import bench
from oracle import circulant_oracle as co
from tests.gpu_util import TOL, row_relerr, to_f64

pytestmark = pytest.mark.gpu


def _inner(a: torch.Tensor, b: torch.Tensor):
    a64, b64 = a.double().flatten(), b.double().flatten()
    scale = float(a64.pow(2).mean().sqrt() * b64.pow(2).mean().sqrt()) * math.sqrt(a64.numel())
    return float((a64 * b64).sum()), scale


def _adjoint(x, dy, y, dx, c=None, dc=None):
    s_y, scale_y = _inner(dy, y)
    s_x, scale_x = _inner(dx, x)
    assert abs(s_y - s_x) <= 2e-2 * max(scale_y, scale_x), (s_y, s_x, scale_y, scale_x)
    if dc is not None:
        s_c, _ = _inner(dc, c)
        assert abs(s_c - s_y) <= 2e-2 * scale_y and abs(s_c - s_x) <= 2e-2 * scale_x, (s_c, s_y, s_x)


def _oracle_check(x, c, dy, y, dx, dc=None):
    p = c.shape[-1]
    xr, cr, dyr = to_f64(x), to_f64(c), to_f64(dy)
    assert row_relerr(to_f64(y), co.circulant_forward_fft(xr, cr)) <= TOL["bf16"]
    dxo, dco = co.circulant_backward_fft(xr, cr, dyr)
    assert row_relerr(to_f64(dx), dxo) <= TOL["bf16"]
    if dc is not None:
        assert row_relerr(to_f64(dc).reshape(-1, p), dco.reshape(-1, p)) <= TOL["f32"]


@pytest.mark.parametrize("spectra", [False, True])
@pytest.mark.parametrize("p", [128, 512, 4096])
def test_single_layer_rotation(p, spectra):
    print(f"bench single layer D=4096 B=256 p={p} spectra={spectra}: one replayed rotation", flush=True)
    w = bench.circ_layer_setup(256, 4096, p, spectra=spectra)
    g = bench._graph(w["rot"])
    for t in w["ys"] + w["dxs"] + [w["dc"]]:
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    n = len(w["xs"])
    assert all(bool(torch.isfinite(t).all()) for t in w["ys"] + w["dxs"] + [w["dc"]])
    for j in range(n):
        last = j == n - 1
        _adjoint(w["xs"][j], w["dys"][j], w["ys"][j], w["dxs"][j], w["c"] if last else None, w["dc"] if last else None)
    _oracle_check(w["xs"][0], w["c"], w["dys"][0], w["ys"][0], w["dxs"][0])
    _oracle_check(w["xs"][-1], w["c"], w["dys"][-1], w["ys"][-1], w["dxs"][-1], w["dc"])


@pytest.mark.parametrize("spectra", [False, True])
def test_adapters_step(spectra):
    print(f"bench 128 adapters 4096x4096 p=1024, 2048 tokens spectra={spectra}: one replayed step", flush=True)
    w = bench.circ_adapters_setup(spectra=spectra)
    g = bench._graph(w["step"])
    for t in w["ys"] + w["dxs"] + w["dcs"]:
        t.fill_(float("nan"))
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    n = len(w["xs"])
    assert n == 128
    assert all(bool(torch.isfinite(t).all()) for t in w["ys"] + w["dxs"] + w["dcs"])
    for a in range(n):
        _adjoint(w["xs"][a], w["dys"][a], w["ys"][a], w["dxs"][a], w["cs"][a], w["dcs"][a])
    for a in (0, 64, 127):
        print(f"  adapter {a} against the oracle", flush=True)
        _oracle_check(w["xs"][a], w["cs"][a], w["dys"][a], w["ys"][a], w["dxs"][a], w["dcs"][a])
