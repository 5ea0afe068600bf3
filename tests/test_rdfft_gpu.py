"""GPU parity of the in-place packed real FFT against the fp64 oracle.

Every case feeds the HIP path (through the C ABI) and the oracle the same
seeded values and compares every row: normwise relative error per row, max
over rows, <= 1e-5 for fp32 storage, <= 2e-2 for bf16 storage and <= 1e-3
for fp16 storage.
"""

import numpy as np
import pytest
import torch

import block_circulant_layers_amd as bcl
from block_circulant_layers_amd import synthetic as syn
from oracle import rdfft_oracle as ro
from tests.gpu_util import TOL, TORCH_DT, device_input, row_relerr, to_f64

pytestmark = pytest.mark.gpu

ALL_P = [2, 4, 8, 16, 32, 64, 128, 256, 512, 1024, 2048, 4096, 8192, 16384, 32768]


def _say(*a):
    print(*a, flush=True)


def _check_fwd_inv(rows, p, dtype, workload=syn.WL_TEST, index=0):
    x, xref = device_input((rows, p), workload, syn.T_X, index, dtype=dtype)
    _say(f"rdfft fwd rows={rows} p={p} dtype={dtype}")
    bcl.rdfft_forward(x)
    torch.cuda.synchronize()
    z = to_f64(x)
    err_f = row_relerr(z, ro.rdfft_forward(xref))
    _say(f"rdfft inv rows={rows} p={p} dtype={dtype}")
    bcl.rdfft_inverse(x)
    torch.cuda.synchronize()
    err_i = row_relerr(to_f64(x), ro.rdfft_inverse(z))
    assert err_f <= TOL[dtype], err_f
    assert err_i <= TOL[dtype], err_i
    return err_f, err_i


@pytest.mark.parametrize("dtype", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("p", ALL_P)
def test_parity_all_lengths(p, dtype):
    # several workgroups plus a ragged tail
    rows = max(3, (3 * 4096) // p) + 5
    _check_fwd_inv(rows, p, dtype, index=p)


@pytest.mark.parametrize("p", ALL_P)
def test_single_row_and_roundtrip(p):
    x, xref = device_input((1, p), syn.WL_TEST, syn.T_X, 100 + p)
    bcl.rdfft_forward(x)
    bcl.rdfft_inverse(x)
    torch.cuda.synchronize()
    assert row_relerr(to_f64(x), xref) <= 1e-5


def test_empty_batch_is_noop():
    x = torch.empty(0, 512, device="cuda:0")
    bcl.rdfft_forward(x)
    bcl.rdfft_inverse(x)
    torch.cuda.synchronize()


@pytest.mark.parametrize("p", [2, 16, 512, 4096, 32768])
def test_closed_forms_on_gpu(p):
    n = np.arange(p)
    rows = np.stack([np.eye(1, p, 0)[0], np.ones(p), (-1.0) ** n, np.cos(2 * np.pi * n / p), np.sin(2 * np.pi * n / p)])
    x = torch.tensor(rows, dtype=torch.float32, device="cuda:0")
    bcl.rdfft_forward(x)
    torch.cuda.synchronize()
    got = to_f64(x)
    want = np.zeros_like(got)
    want[0, : p // 2 + 1] = 1.0
    want[1, 0] = p
    want[2, p // 2] = p
    if p > 2:
        want[3, 1] = p / 2
        want[4, p - 1] = -p / 2
    else:  # p = 2: cos(pi n) = (-1)^n, sin(pi n) = 0
        want[3, 1] = p
    assert np.allclose(got, want, atol=2e-6 * p)


@pytest.mark.parametrize("rows,p,dtype", [(65539, 128, "f32"), (65539, 128, "bf16"), (131075, 32, "f16"),
                                          (40001, 256, "bf16"), (20003, 512, "f32"), (9001, 1024, "f32"),
                                          (4099, 4096, "bf16")])
def test_persistent_row_groups(rows, p, dtype):
    # more row groups than resident workgroups (256 CUs x 8 one-wave workgroups
    # of 64 / T rows for p <= 512): every workgroup loops over several groups,
    # prefetching the next, and the last group is ragged
    _check_fwd_inv(rows, p, dtype, index=rows)


@pytest.mark.parametrize("p", [128, 4096, 16384])
def test_inverse_accepts_any_packed_vector(p):
    z, zref = device_input((64, p), syn.WL_TEST, syn.T_DY, p)
    bcl.rdfft_inverse(z)
    torch.cuda.synchronize()
    assert row_relerr(to_f64(z), ro.rdfft_inverse(zref)) <= 1e-5


@pytest.mark.parametrize("p,dtype", [(512, "f32"), (4096, "bf16"), (32768, "f32")])
def test_bitwise_deterministic(p, dtype):
    x, _ = device_input((1024, p), syn.WL_TEST, syn.T_X, 7, dtype=dtype)
    outs = []
    for _ in range(10):
        y = x.clone()
        bcl.rdfft_forward(y)
        outs.append(y)
    torch.cuda.synchronize()
    for y in outs[1:]:
        assert torch.equal(y, outs[0])
    for y in outs:
        bcl.rdfft_inverse(y)
    torch.cuda.synchronize()
    for y in outs[1:]:
        assert torch.equal(y, outs[0])


def test_stream_argument():
    s = torch.cuda.Stream()
    x, xref = device_input((256, 1024), syn.WL_TEST, syn.T_X, 11)
    with torch.cuda.stream(s):
        bcl.rdfft_forward(x)
    s.synchronize()
    assert row_relerr(to_f64(x), ro.rdfft_forward(xref)) <= 1e-5


# ---- the benchmark workloads at full size, in the launch configuration timed ----


def test_workload_4096x512_f32_roundtrip():
    # 4096 rows of 512, fp32, forward then inverse in place, every row checked
    ef, ei = _check_fwd_inv(4096, 512, "f32", syn.WL_RDFFT_512)
    _say(f"4096x512 f32: fwd {ef:.2e} inv {ei:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_workload_4096x4096(dtype):
    ef, ei = _check_fwd_inv(4096, 4096, dtype, syn.WL_RDFFT_LARGE)
    _say(f"4096x4096 {dtype}: fwd {ef:.2e} inv {ei:.2e}")


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_workload_16384x128(dtype):
    ef, ei = _check_fwd_inv(16384, 128, dtype, syn.WL_RDFFT_LARGE, index=1)
    _say(f"16384x128 {dtype}: fwd {ef:.2e} inv {ei:.2e}")


@pytest.mark.parametrize("rows,p", [(2048, 8192), (512, 32768)])
def test_long_rows_64mib(rows, p):
    # 64 MiB of fp32 rows longer than 4096: one workgroup per row
    ef, ei = _check_fwd_inv(rows, p, "f32", syn.WL_RDFFT_LARGE, index=p)
    _say(f"{rows}x{p} f32: fwd {ef:.2e} inv {ei:.2e}")


def test_no_device_allocation():
    # zero workspace: the library allocates nothing; torch's allocator sees no growth
    x, _ = device_input((4096, 4096), syn.WL_TEST, syn.T_X, 3)
    torch.cuda.synchronize()
    torch.cuda.reset_peak_memory_stats()
    before = torch.cuda.memory_allocated()
    free0, _ = torch.cuda.mem_get_info()
    bcl.rdfft_forward(x)
    bcl.rdfft_inverse(x)
    torch.cuda.synchronize()
    free1, _ = torch.cuda.mem_get_info()
    assert torch.cuda.max_memory_allocated() == before
    assert free1 >= free0 - (2 << 20)  # no device allocation behind torch's back (2 MiB slack)
