"""The library's host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

The same host build as the LDS schedule check (tests/lds_check: rdfft_lib.hip
for the host against a CPU stand-in of the HIP runtime), compiled with
-fsanitize=address,undefined and no recovery: any out-of-bounds access, signed
overflow, invalid shift or misaligned access in the argument checks
(rdfft_validate.hpp), the dispatch and grid arithmetic of rdfft_lib.hip or the
kernels aborts the run.  It runs every argument case of tests/abi_cases.py
(the cases test_abi_cpu.py sends to the built library), including sizes at
the int64 limit, and a few real calls whose outputs are checked against the
fp64 oracle."""

from __future__ import annotations

import os
import re
import subprocess

import numpy as np
import pytest

from block_circulant_layers_amd import synthetic as syn
from oracle import circulant_oracle as co
from oracle import rdfft_oracle as ro
from tests import abi_cases
from tests.lds_check import build_emu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ENV = dict(os.environ, EMU_CUS="1", ASAN_OPTIONS="detect_leaks=0:abort_on_error=0:exitcode=67",
           UBSAN_OPTIONS="halt_on_error=1:print_stacktrace=1:exitcode=68")


def _status_codes():
    hdr = open(os.path.join(ROOT, "include", "rdfft.h")).read()
    d = {k: int(v) for k, v in re.findall(r"#define\s+(RDFFT_\w+)\s+(\d+)", hdr)}
    return {"OK": d["RDFFT_OK"], "NULL": d["RDFFT_ERR_NULL"], "SIZE": d["RDFFT_ERR_SIZE"],
            "SHAPE": d["RDFFT_ERR_SHAPE"], "DTYPE": d["RDFFT_ERR_DTYPE"], "ALIGN": d["RDFFT_ERR_ALIGN"],
            "ALIAS": d["RDFFT_ERR_ALIAS"], "SCRATCH": d["RDFFT_ERR_SCRATCH"]}


@pytest.fixture(scope="module")
def exe():
    return build_emu.build("asan")


def _check_clean(r):
    assert "AddressSanitizer" not in r.stderr and "runtime error" not in r.stderr, r.stderr[:4000]
    assert r.returncode == 0, r.stderr[-4000:]


def test_argument_cases(exe):
    codes = _status_codes()
    lines = []
    for fn, args, _ in abi_cases.CASES:
        lines.append(" ".join([fn] + ["null" if a is None else str(a) for a in args]))
    r = subprocess.run([exe, "cases"], input="\n".join(lines) + "\n", capture_output=True, text=True, env=ENV,
                       timeout=300)
    _check_clean(r)
    got = [int(v) for v in r.stdout.split()[: len(lines)]]
    want = [codes[e] for _, _, e in abi_cases.CASES]
    bad = [(abi_cases.CASES[i], g) for i, (g, w) in enumerate(zip(got, want)) if g != w]
    assert len(got) == len(want) and not bad, bad


def _write(path, t):
    import torch

    t.contiguous().view(torch.int16 if t.dtype != torch.float32 else torch.float32).numpy().tofile(path)


def _read(path, shape, dt):
    import torch

    if dt == "f32":
        return np.fromfile(path, dtype=np.float32).reshape(shape).astype(np.float64)
    raw = torch.from_numpy(np.fromfile(path, dtype=np.int16).reshape(shape))
    return raw.view(torch.bfloat16 if dt == "bf16" else torch.float16).to(torch.float64).numpy()


def _relerr(got, want):
    got, want = got.reshape(-1, got.shape[-1]), want.reshape(-1, want.shape[-1])
    return float(np.max(np.linalg.norm(got - want, axis=1) / np.linalg.norm(want, axis=1)))


@pytest.mark.parametrize("rows,p,dt", [(35, 512, "f32"), (3, 16384, "bf16"), (517, 32, "f16")])
def test_transform_calls(exe, tmp_path, rows, p, dt):
    t, xr = syn.cast_like_device(syn.normal((rows, p), syn.WL_TEST, syn.T_X, 40 + p), dt)
    f = str(tmp_path / "d")
    _write(f, t)
    r = subprocess.run([exe, "fwd", str(rows), str(p), str({"f32": 0, "bf16": 1, "f16": 2}[dt]), f],
                       capture_output=True, text=True, env=ENV, timeout=300)
    _check_clean(r)
    assert _relerr(_read(f, (rows, p), dt), ro.rdfft_forward(xr)) <= {"f32": 1e-5, "bf16": 2e-2, "f16": 1e-3}[dt]


@pytest.mark.parametrize("batch,d_in,d_out,p", [(5, 64, 48, 16), (3, 512, 1024, 256), (4, 640, 384, 128)])
def test_circulant_calls(exe, tmp_path, batch, d_in, d_out, p):
    q, k = d_out // p, d_in // p
    xt, xr = syn.cast_like_device(syn.normal((batch, d_in), syn.WL_TEST, syn.T_X, 60 + p), "f32")
    ct, cr = syn.cast_like_device(syn.normal((q, k, p), syn.WL_TEST, syn.T_C, 60 + p), "f32")
    gt, gr = syn.cast_like_device(syn.normal((batch, d_out), syn.WL_TEST, syn.T_DY, 60 + p), "f32")
    fx, fc, fg, fy, fdx, fdc = (str(tmp_path / n) for n in ("x", "c", "dy", "y", "dx", "dc"))
    _write(fx, xt)
    _write(fc, ct)
    _write(fg, gt)
    dims = [str(v) for v in (batch, d_in, d_out, p, 0)]
    r = subprocess.run([exe, "circ_fwd", *dims, fx, fc, fy], capture_output=True, text=True, env=ENV, timeout=300)
    _check_clean(r)
    assert _relerr(_read(fy, (batch, d_out), "f32"), co.circulant_forward_dense(xr, cr)) <= 1e-5
    r = subprocess.run([exe, "circ_bwd", *dims, fx, fc, fg, fdx, fdc], capture_output=True, text=True, env=ENV,
                       timeout=300)
    _check_clean(r)
    dxo, dco = co.circulant_backward_dense(xr, cr, gr)
    assert _relerr(_read(fdx, (batch, d_in), "f32"), dxo) <= 1e-5
    assert _relerr(_read(fdc, (q * k, p), "f32"), dco.reshape(q * k, p)) <= 1e-5
    # the deterministic dc (workspace slices summed in order)
    r = subprocess.run([exe, "circ_det", *dims, fx, fc, fg, fdx, fdc], capture_output=True, text=True, env=ENV,
                       timeout=300)
    _check_clean(r)
    assert _relerr(_read(fdx, (batch, d_in), "f32"), dxo) <= 1e-5
    assert _relerr(_read(fdc, (q * k, p), "f32"), dco.reshape(q * k, p)) <= 1e-5
    # the zeroing forward and the accumulating backward (twice)
    r = subprocess.run([exe, "circ_step", *dims, fx, fc, fg, fy, fdx, fdc], capture_output=True, text=True, env=ENV,
                       timeout=300)
    _check_clean(r)
    assert _relerr(_read(fy, (batch, d_out), "f32"), co.circulant_forward_dense(xr, cr)) <= 1e-5
    assert _relerr(_read(fdx, (batch, d_in), "f32"), dxo) <= 1e-5
    assert _relerr(_read(fdc, (q * k, p), "f32"), 2 * dco.reshape(q * k, p)) <= 1e-5
    # the weights given as spectra: circulant_fwd_step, circulant_weight_spectra,
    # circulant_fwd_spec and circulant_bwd_spec
    fy2, fcs = str(tmp_path / "y2"), str(tmp_path / "cs")
    r = subprocess.run([exe, "circ_spec", *dims, fx, fc, fg, fy, fy2, fdx, fdc, fcs], capture_output=True, text=True,
                       env=ENV, timeout=300)
    _check_clean(r)
    assert _relerr(_read(fcs, (q * k, p), "f32"), ro.rdfft_forward(cr.reshape(q * k, p))) <= 1e-5
    assert _relerr(_read(fy, (batch, d_out), "f32"), co.circulant_forward_dense(xr, cr)) <= 1e-5
    assert _relerr(_read(fy2, (batch, d_out), "f32"), co.circulant_forward_dense(xr, cr)) <= 1e-5
    assert _relerr(_read(fdx, (batch, d_in), "f32"), dxo) <= 1e-5
    assert _relerr(_read(fdc, (q * k, p), "f32"), 2 * dco.reshape(q * k, p)) <= 1e-5
