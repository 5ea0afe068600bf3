"""LDS schedule check of every kernel on the CPU, under ThreadSanitizer.

The library (rdfft_lib.hip: C ABI, dispatch and kernels) is built for the host
against the CPU stand-in of hip/hip_runtime.h in tests/lds_check: each GPU
thread of a workgroup runs as a host thread and __syncthreads() is a barrier
of those threads.  ThreadSanitizer then reports any two threads that touch one
LDS (or global) location between two barriers with at least one write: a
missing barrier, or two threads of one pass owning the same slot.  The passes
checked this way are the per-stage group partitions of the packed transform
(Paper-Notes page, section "四元素对称群 (Proposition 1)") as the kernels
schedule them, several stages per pass, with their padded exchange layouts,
plus the block-circulant tiles (section "循环矩阵训练适配").

Each case also compares the emulated outputs with the fp64 oracle, at the
GPU parity gates, so the host build is known to run the same arithmetic.
Shapes are small but make the persistent kernels loop over several row groups
with a ragged last one (the stand-in reports 1 compute unit, so grids are
small), and cover every transform length, the circulant paths (token-
persistent tiles, one-launch backward, small-p kernels) for each p, 2D and the
spectrum utilities.
"""

from __future__ import annotations

import os
import subprocess

import numpy as np
import pytest

from block_circulant_layers_amd import synthetic as syn
from oracle import circulant_oracle as co
from oracle import rdfft2d_oracle as r2
from oracle import rdfft_oracle as ro
from tests.lds_check import build_emu

DT = {"f32": 0, "bf16": 1, "f16": 2}
TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 1e-3}
ENV = dict(os.environ, EMU_CUS="1", TSAN_OPTIONS="halt_on_error=1 exitcode=66 report_signal_unsafe=0")


@pytest.fixture(scope="module")
def exe():
    return build_emu.build("tsan")


def _run(exe, *args):
    r = subprocess.run([exe, *map(str, args)], capture_output=True, text=True, env=ENV, timeout=600)
    assert "ThreadSanitizer" not in r.stderr, r.stderr[:4000]
    assert r.returncode == 0, r.stderr[-4000:]
    status = int(r.stdout.split()[1])
    assert status == 0, r.stdout
    return r.stdout


def _write(path, t):
    import torch

    raw = t.contiguous().view(torch.int16 if t.dtype != torch.float32 else torch.float32).numpy()
    raw.tofile(path)


def _read(path, shape, dt):
    import torch

    if dt == "f32":
        return np.fromfile(path, dtype=np.float32).reshape(shape).astype(np.float64)
    raw = torch.from_numpy(np.fromfile(path, dtype=np.int16).reshape(shape))
    return raw.view(torch.bfloat16 if dt == "bf16" else torch.float16).to(torch.float64).numpy()


def _relerr(got, want):
    got = got.reshape(-1, got.shape[-1])
    want = want.reshape(-1, want.shape[-1])
    den = np.linalg.norm(want, axis=1)
    return float(np.max(np.linalg.norm(got - want, axis=1) / np.where(den == 0, 1, den)))


def test_checker_reports_a_missing_barrier(exe):
    r = subprocess.run([exe, "selftest", "race"], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 66 and "ThreadSanitizer: data race" in r.stderr
    r = subprocess.run([exe, "selftest", "ok"], capture_output=True, text=True, env=ENV, timeout=120)
    assert r.returncode == 0 and "ThreadSanitizer" not in r.stderr, r.stderr[:2000]


# rows per length: a few row groups per persistent workgroup and a ragged last group
# (rows of 16384 and 32768: one workgroup per row)
RDFFT_CASES = [(2, 1027, "f32"), (4, 1029, "f32"), (8, 1030, "f32"), (16, 1031, "f32"), (32, 517, "f32"),
               (64, 261, "f32"), (128, 133, "f32"), (256, 69, "f32"), (512, 35, "f32"), (1024, 19, "f32"),
               (2048, 11, "f32"), (4096, 5, "f32"), (8192, 5, "f32"), (16384, 2, "f32"), (32768, 2, "f32"),
               (16384, 5, "bf16"), (32768, 3, "f16"),
               (128, 133, "bf16"), (256, 69, "f16"), (512, 35, "bf16"), (1024, 19, "bf16"), (4096, 9, "bf16"),
               (4096, 9, "f16"), (8192, 5, "bf16")]


@pytest.mark.parametrize("p,rows,dt", RDFFT_CASES)
def test_transforms(exe, tmp_path, p, rows, dt):
    t, xr = syn.cast_like_device(syn.normal((rows, p), syn.WL_TEST, syn.T_X, 900 + p), dt)
    f = str(tmp_path / "d.bin")
    _write(f, t)
    _run(exe, "fwd", rows, p, DT[dt], f)
    z = _read(f, (rows, p), dt)
    assert _relerr(z, ro.rdfft_forward(xr)) <= TOL[dt]
    _run(exe, "inv", rows, p, DT[dt], f)
    assert _relerr(_read(f, (rows, p), dt), ro.rdfft_inverse(z)) <= TOL[dt]


# (batch, d_in, d_out, p, dtype): small-p kernels, token-persistent tiles and
# the one-launch backward at every p, rectangular weights, ragged token ranges
CIRC_CASES = [(5, 64, 48, 16, "f32"), (3, 96, 64, 32, "bf16"), (7, 256, 192, 64, "bf16"), (9, 512, 512, 128, "bf16"),
              (5, 512, 1024, 256, "f32"), (6, 1024, 1024, 512, "bf16"), (5, 2048, 4096, 1024, "bf16"),
              (3, 4096, 4096, 2048, "f32"), (5, 4096, 4096, 4096, "bf16"), (2, 8192, 4096, 4096, "f16")]


@pytest.mark.parametrize("batch,d_in,d_out,p,dt", CIRC_CASES)
def test_circulant(exe, tmp_path, batch, d_in, d_out, p, dt):
    q, k = d_out // p, d_in // p
    xt, xr = syn.cast_like_device(syn.normal((batch, d_in), syn.WL_TEST, syn.T_X, 950 + p), dt)
    ct, cr = syn.cast_like_device(syn.normal((q, k, p), syn.WL_TEST, syn.T_C, 950 + p, d_in**-0.5), "f32")
    gt, gr = syn.cast_like_device(syn.normal((batch, d_out), syn.WL_TEST, syn.T_DY, 950 + p), dt)
    fx, fc, fg = str(tmp_path / "x"), str(tmp_path / "c"), str(tmp_path / "dy")
    fy, fdx, fdc = str(tmp_path / "y"), str(tmp_path / "dx"), str(tmp_path / "dc")
    _write(fx, xt)
    _write(fc, ct)
    _write(fg, gt)
    _run(exe, "circ_fwd", batch, d_in, d_out, p, DT[dt], fx, fc, fy)
    assert _relerr(_read(fy, (batch, d_out), dt), co.circulant_forward_fft(xr, cr)) <= TOL[dt]
    dxo, dco = co.circulant_backward_fft(xr, cr, gr)
    # both outputs (one launch where the length allows), then each alone
    for want_dx, want_dc in ((True, True), (True, False), (False, True)):
        _run(exe, "circ_bwd", batch, d_in, d_out, p, DT[dt], fx, fc, fg, fdx if want_dx else "-",
             fdc if want_dc else "-")
        if want_dx:
            assert _relerr(_read(fdx, (batch, d_in), dt), dxo) <= TOL[dt]
        if want_dc:
            assert _relerr(_read(fdc, (q * k, p), "f32"), dco.reshape(q * k, p)) <= TOL["f32"]


# a training step as the layer runs it: circulant_fwd_zero clears a dc that
# holds garbage, then circulant_bwd_acc adds twice (dc = 2 x the gradient).
# Paths: small p (fill after the forward, spectra added into dc), the
# one-launch backward (time-domain adds), and dc without dx at p = 128
# (packed spectra: old dc transformed forward first) and at p = 256.
STEP_CASES = [(5, 64, 48, 16, "f32", True), (4, 96, 64, 32, "f32", False), (9, 512, 512, 128, "bf16", True),
              (9, 512, 512, 128, "bf16", False), (5, 512, 1024, 256, "f32", False),
              (5, 4096, 4096, 4096, "bf16", True)]


@pytest.mark.parametrize("batch,d_in,d_out,p,dt,want_dx", STEP_CASES)
def test_circulant_step(exe, tmp_path, batch, d_in, d_out, p, dt, want_dx):
    q, k = d_out // p, d_in // p
    xt, xr = syn.cast_like_device(syn.normal((batch, d_in), syn.WL_TEST, syn.T_X, 960 + p), dt)
    ct, cr = syn.cast_like_device(syn.normal((q, k, p), syn.WL_TEST, syn.T_C, 960 + p, d_in**-0.5), "f32")
    gt, gr = syn.cast_like_device(syn.normal((batch, d_out), syn.WL_TEST, syn.T_DY, 960 + p), dt)
    fx, fc, fg = str(tmp_path / "x"), str(tmp_path / "c"), str(tmp_path / "dy")
    fy, fdx, fdc = str(tmp_path / "y"), str(tmp_path / "dx"), str(tmp_path / "dc")
    _write(fx, xt)
    _write(fc, ct)
    _write(fg, gt)
    _run(exe, "circ_step", batch, d_in, d_out, p, DT[dt], fx, fc, fg, fy, fdx if want_dx else "-", fdc)
    assert _relerr(_read(fy, (batch, d_out), dt), co.circulant_forward_fft(xr, cr)) <= TOL[dt]
    dxo, dco = co.circulant_backward_fft(xr, cr, gr)
    if want_dx:
        assert _relerr(_read(fdx, (batch, d_in), dt), dxo) <= TOL[dt]
    assert _relerr(_read(fdc, (q * k, p), "f32"), 2 * dco.reshape(q * k, p)) <= TOL["f32"]


# the weights given as spectra: circulant_fwd_step (y, cs, and a dc that held
# garbage cleared), circulant_weight_spectra (bitwise the cs of the forward,
# checked by the driver), circulant_fwd_spec from cs, circulant_bwd_spec
# overwriting dc, then adding into it (dc = 2 x the gradient).  Routes: the small-p kernels (p < 64
# and p = 128 with 40 input blocks, more than one transform round holds), the
# token-persistent tiles and the one-launch backward at every p from 64 to
# 4096, output tiles past the last block (q = 3 and k = 5 at p = 128), and dc
# without dx.
SPEC_CASES = [(5, 64, 48, 16, "f32", True), (4, 96, 64, 32, "f32", False), (7, 256, 192, 64, "bf16", True),
              (9, 640, 384, 128, "bf16", True), (9, 640, 384, 128, "bf16", False), (3, 5120, 384, 128, "f32", True),
              (5, 512, 1024, 256, "f32", True), (6, 1024, 1536, 512, "bf16", True), (5, 2048, 4096, 1024, "bf16", True),
              (3, 4096, 2048, 2048, "f32", True), (5, 4096, 4096, 4096, "bf16", True),
              (2, 8192, 4096, 4096, "f16", False)]


@pytest.mark.parametrize("batch,d_in,d_out,p,dt,want_dx", SPEC_CASES)
def test_circulant_spec(exe, tmp_path, batch, d_in, d_out, p, dt, want_dx):
    q, k = d_out // p, d_in // p
    xt, xr = syn.cast_like_device(syn.normal((batch, d_in), syn.WL_TEST, syn.T_X, 990 + p), dt)
    ct, cr = syn.cast_like_device(syn.normal((q, k, p), syn.WL_TEST, syn.T_C, 990 + p, d_in**-0.5), "f32")
    gt, gr = syn.cast_like_device(syn.normal((batch, d_out), syn.WL_TEST, syn.T_DY, 990 + p), dt)
    fx, fc, fg = str(tmp_path / "x"), str(tmp_path / "c"), str(tmp_path / "dy")
    fy, fdx, fdc = str(tmp_path / "y"), str(tmp_path / "dx"), str(tmp_path / "dc")
    fy2, fcs = str(tmp_path / "y2"), str(tmp_path / "cs")
    _write(fx, xt)
    _write(fc, ct)
    _write(fg, gt)
    _run(exe, "circ_spec", batch, d_in, d_out, p, DT[dt], fx, fc, fg, fy, fy2, fdx if want_dx else "-", fdc, fcs)
    assert _relerr(_read(fcs, (q * k, p), "f32"), ro.rdfft_forward(cr.reshape(q * k, p))) <= TOL["f32"]
    yo = co.circulant_forward_fft(xr, cr)
    assert _relerr(_read(fy, (batch, d_out), dt), yo) <= TOL[dt]
    assert _relerr(_read(fy2, (batch, d_out), dt), yo) <= TOL[dt]
    dxo, dco = co.circulant_backward_fft(xr, cr, gr)
    if want_dx:
        assert _relerr(_read(fdx, (batch, d_in), dt), dxo) <= TOL[dt]
    assert _relerr(_read(fdc, (q * k, p), "f32"), 2 * dco.reshape(q * k, p)) <= TOL["f32"]


# the deterministic dc (workspace slices summed in order) on every route:
# small-p kernels, token-persistent dc alone with packed-spectra slices (p = 64,
# 128) and time-domain slices (p = 256), and the one-launch backward with dx
DET_CASES = [(5, 64, 48, 16, "f32", True), (4, 96, 64, 32, "f32", False), (7, 256, 192, 64, "bf16", False),
             (9, 512, 512, 128, "bf16", False), (5, 512, 1024, 256, "f32", False), (9, 512, 512, 128, "bf16", True),
             (5, 2048, 4096, 1024, "bf16", True), (5, 4096, 4096, 4096, "bf16", True)]


@pytest.mark.parametrize("batch,d_in,d_out,p,dt,want_dx", DET_CASES)
def test_circulant_det(exe, tmp_path, batch, d_in, d_out, p, dt, want_dx):
    q, k = d_out // p, d_in // p
    xt, xr = syn.cast_like_device(syn.normal((batch, d_in), syn.WL_TEST, syn.T_X, 980 + p), dt)
    ct, cr = syn.cast_like_device(syn.normal((q, k, p), syn.WL_TEST, syn.T_C, 980 + p, d_in**-0.5), "f32")
    gt, gr = syn.cast_like_device(syn.normal((batch, d_out), syn.WL_TEST, syn.T_DY, 980 + p), dt)
    fx, fc, fg = str(tmp_path / "x"), str(tmp_path / "c"), str(tmp_path / "dy")
    fdx, fdc = str(tmp_path / "dx"), str(tmp_path / "dc")
    _write(fx, xt)
    _write(fc, ct)
    _write(fg, gt)
    _run(exe, "circ_det", batch, d_in, d_out, p, DT[dt], fx, fc, fg, fdx if want_dx else "-", fdc)
    dxo, dco = co.circulant_backward_fft(xr, cr, gr)
    if want_dx:
        assert _relerr(_read(fdx, (batch, d_in), dt), dxo) <= TOL[dt]
    assert _relerr(_read(fdc, (q * k, p), "f32"), dco.reshape(q * k, p)) <= TOL["f32"]


@pytest.mark.parametrize("n,h,w,dt", [(2, 16, 32, "f32"), (1, 64, 512, "bf16"), (1, 4096, 16, "f32"),
                                      (1, 512, 64, "f16"), (3, 8, 8, "f32")])
def test_2d(exe, tmp_path, n, h, w, dt):
    t, xr = syn.cast_like_device(syn.normal((n, h, w), syn.WL_TEST, syn.T_X, 970 + h + w), dt)
    f = str(tmp_path / "d.bin")
    _write(f, t)
    _run(exe, "fwd2d", n, h, w, DT[dt], f)
    z = _read(f, (n, h, w), dt)
    tol = {"f32": 1e-5, "bf16": 2e-2, "f16": 3e-3}[dt]
    assert _relerr(z, r2.rdfft2d_forward(xr)) <= tol
    _run(exe, "inv2d", n, h, w, DT[dt], f)
    assert _relerr(_read(f, (n, h, w), dt), r2.rdfft2d_inverse(z)) <= tol


@pytest.mark.parametrize("rows,p,dt", [(37, 512, "f32"), (5, 4096, "bf16"), (300, 2, "f16")])
def test_spectrum(exe, tmp_path, rows, p, dt):
    t, zr = syn.cast_like_device(syn.normal((rows, p), syn.WL_TEST, syn.T_X, 990 + p), dt)
    fz, fs, fz2 = str(tmp_path / "z"), str(tmp_path / "s"), str(tmp_path / "z2")
    _write(fz, t)
    _run(exe, "unpack", rows, p, DT[dt], fz, fs)
    spec = np.fromfile(fs, dtype=np.float32).reshape(rows, p // 2 + 1, 2).astype(np.float64)
    want = ro.unpack_spectrum(zr)[:, : p // 2 + 1]
    assert np.array_equal(spec[..., 0], want.real) and np.array_equal(spec[..., 1], want.imag)
    _run(exe, "pack", rows, p, DT[dt], fs, fz2)
    assert np.array_equal(_read(fz2, (rows, p), dt), zr)
