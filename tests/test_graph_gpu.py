"""Launches captured in a HIP graph give the eager results on every replay.

The library's calls only enqueue kernels (no allocation, no memset), so they can
be captured.  Each graph is replayed several times with eager work and
synchronisations in between, and every replay is checked against the eager
result: bit-exact for the transforms, within the fp32 gate for dc (its token
sum is accumulated atomically, so its last bits may vary).
"""

import pytest
import torch

import block_circulant_layers_amd as bcl
from block_circulant_layers_amd import synthetic as syn
from tests.gpu_util import device_input

pytestmark = pytest.mark.gpu


def _capture(fn):
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def test_transform_graph_replays():
    x0, _ = device_input((300, 512), syn.WL_TEST, syn.T_X, 31)
    eager = x0.clone()
    bcl.rdfft_forward(eager)
    buf = x0.clone()
    g = _capture(lambda: bcl.rdfft_forward(buf))
    for i in range(4):
        buf.copy_(x0)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf, eager), i


# p = 128 and 4096: dx and dc in one launch (at 4096 with a wider dx tile than
# the forward's); p = 16: the small-p kernels
@pytest.mark.parametrize("b,d,p", [(64, 1024, 128), (32, 4096, 4096), (24, 256, 16)])
def test_circulant_graph_replays(b, d, p):
    x, _ = device_input((b, d), syn.WL_TEST, syn.T_X, 32, dtype="bf16")
    c, _ = device_input((d // p, d // p, p), syn.WL_TEST, syn.T_C, 32, scale=1 / 32)
    dy, _ = device_input((b, d), syn.WL_TEST, syn.T_DY, 32, dtype="bf16")
    y0 = bcl.circulant_fwd(x, c)
    dx0, dc0 = bcl.circulant_bwd(x, c, dy)
    y, dx, dc = torch.empty_like(y0), torch.empty_like(dx0), torch.empty_like(dc0)

    def step():
        bcl.circulant_fwd(x, c, y)
        bcl.circulant_bwd(x, c, dy, dx=dx, dc=dc)

    g = _capture(step)
    for i in range(4):
        for t in (y, dx, dc):
            t.fill_(float("nan"))  # eager work; the replay must overwrite everything
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0) and torch.equal(dx, dx0), i
        err = float((dc - dc0).norm() / dc0.norm())
        assert err <= 1e-5, (i, err)


# the training-step calls: the forward clears dc in its launch (p = 128, 4096),
# or with a fill kernel (p = 16); the backward adds into it, in the time domain
# (one launch with dx) or as packed spectra after transforming dc (p = 64 without dx)
@pytest.mark.parametrize("b,d,p,want_dx", [(64, 1024, 128, True), (32, 4096, 4096, True), (24, 256, 16, True),
                                           (40, 512, 64, False)])
def test_training_step_graph_replays(b, d, p, want_dx):
    x, _ = device_input((b, d), syn.WL_TEST, syn.T_X, 34, dtype="bf16")
    c, _ = device_input((d // p, d // p, p), syn.WL_TEST, syn.T_C, 34, scale=1 / 32)
    dy, _ = device_input((b, d), syn.WL_TEST, syn.T_DY, 34, dtype="bf16")
    y0 = bcl.circulant_fwd(x, c)
    dx0, dc0 = bcl.circulant_bwd(x, c, dy, need_dx=want_dx)
    y, dc = torch.empty_like(y0), torch.empty_like(dc0)
    dx = torch.empty_like(x) if want_dx else None

    def step():
        bcl.circulant_fwd_zero(x, c, dc, y)
        bcl.circulant_bwd_acc(x, c, dy, dc, dx=dx, need_dx=want_dx)

    g = _capture(step)
    for i in range(4):
        for t in (y, dx, dc):
            if t is not None:
                t.fill_(float("nan"))  # eager work; the replay must clear or overwrite everything
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(y, y0), i
        if want_dx:
            assert torch.equal(dx, dx0), i
        err = float((dc - dc0).norm() / dc0.norm())
        assert err <= 1e-5, (i, err)


# the training step with the weights as spectra: circulant_fwd_step writes cs
# (in its launch at p = 128 and 4096, with a launch of its own at p = 16) and
# clears dc; circulant_bwd_spec reads cs and adds into dc
@pytest.mark.parametrize("b,d,p,want_dx", [(64, 1024, 128, True), (32, 4096, 4096, True), (24, 256, 16, True),
                                           (40, 512, 64, False)])
def test_spectral_step_graph_replays(b, d, p, want_dx):
    x, _ = device_input((b, d), syn.WL_TEST, syn.T_X, 36, dtype="bf16")
    c, _ = device_input((d // p, d // p, p), syn.WL_TEST, syn.T_C, 36, scale=1 / 32)
    dy, _ = device_input((b, d), syn.WL_TEST, syn.T_DY, 36, dtype="bf16")
    cs0 = bcl.circulant_weight_spectra(c)
    y0 = bcl.circulant_fwd(x, c)  # circulant_fwd_step's y is circulant_fwd's
    dx0, dc0 = bcl.circulant_bwd_spec(x, cs0, dy, need_dx=want_dx)
    y, dc, cs = torch.empty_like(y0), torch.empty_like(dc0), torch.empty_like(cs0)
    dx = torch.empty_like(x) if want_dx else None

    def step():
        bcl.circulant_fwd_step(x, c, cs, y, dc=dc)
        bcl.circulant_bwd_spec(x, cs, dy, dx=dx, dc=dc, need_dx=want_dx, accumulate=True)

    g = _capture(step)
    for i in range(4):
        for t in (y, dx, dc, cs):
            if t is not None:
                t.fill_(float("nan"))  # eager work; the replay must clear or overwrite everything
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(cs, cs0) and torch.equal(y, y0), i
        if want_dx:
            assert torch.equal(dx, dx0), i
        err = float((dc - dc0).norm() / dc0.norm())
        assert err <= 1e-5, (i, err)


@pytest.mark.parametrize("b,d,p,want_dx", [(64, 1024, 128, True), (24, 256, 16, True), (40, 512, 64, False)])
def test_deterministic_dc_graph_replays(b, d, p, want_dx):
    # circulant_bwd_det captured: every replay gives the eager result bit for bit
    x, _ = device_input((b, d), syn.WL_TEST, syn.T_X, 35, dtype="bf16")
    c, _ = device_input((d // p, d // p, p), syn.WL_TEST, syn.T_C, 35, scale=1 / 32)
    dy, _ = device_input((b, d), syn.WL_TEST, syn.T_DY, 35, dtype="bf16")
    ws = torch.empty(bcl.circulant_bwd_det_workspace(b, d, d, p, want_dx) // 4, device="cuda:0")
    dx0, dc0 = bcl.circulant_bwd_det(x, c, dy, ws=ws, need_dx=want_dx)
    dc = torch.empty_like(dc0)
    dx = torch.empty_like(x) if want_dx else None
    g = _capture(lambda: bcl.circulant_bwd_det(x, c, dy, dx=dx, dc=dc, ws=ws, need_dx=want_dx))
    for i in range(4):
        for t in (dx, dc, ws):
            if t is not None:
                t.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(dc, dc0), i
        if want_dx:
            assert torch.equal(dx, dx0), i


def test_2d_and_spectrum_graph_replays():
    x0, _ = device_input((2, 256, 512), syn.WL_TEST, syn.T_X, 33)
    eager = x0.clone()
    bcl.rdfft2d_forward(eager)
    spec0 = bcl.rdfft_unpack(eager)
    back0 = torch.empty_like(eager)
    bcl.rdfft_pack(spec0, back0)
    buf, spec, back = x0.clone(), torch.empty_like(spec0), torch.empty_like(back0)

    def step():
        bcl.rdfft2d_forward(buf)
        bcl.rdfft_unpack(buf, spec)
        bcl.rdfft_pack(spec, back)

    g = _capture(step)
    for i in range(4):
        buf.copy_(x0)  # eager work between replays
        spec.fill_(float("nan"))
        back.fill_(float("nan"))
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(buf, eager) and torch.equal(spec, spec0) and torch.equal(back, back0), i
    assert torch.equal(back0, eager)  # pack undoes unpack exactly
