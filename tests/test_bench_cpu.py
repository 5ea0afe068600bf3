"""Host-side checks of bench.py's helpers (no GPU).

The torch.fft forms that bench.py times beside the layer as context must be
the same linear map as the block-circulant layer (Paper-Notes, "循环矩阵训练
适配"): checked here against the oracle's dense forward and backward in float64.
Also: the algorithmic byte and flop counts of the layer workloads, the split of
the timed steps into runs (exactly the requested count), the exit of a
multi-GPU request, and the window and allocation count of the HIP API summary.
"""
import os

import numpy as np
import pytest
import torch

import bench
from oracle import circulant_oracle as co


@pytest.mark.parametrize("real", [True, False])
@pytest.mark.parametrize("shape", [(3, 2, 4, 16), (2, 3, 2, 8), (1, 1, 1, 2)])
def test_torch_fft_context_forms_match_oracle(real, shape):
    b, q, k, p = shape
    rng = np.random.default_rng(5)
    x = rng.standard_normal((b, k * p))
    c = rng.standard_normal((q, k, p))
    dy = rng.standard_normal((b, q * p))
    xt = torch.tensor(x, requires_grad=True)
    ct = torch.tensor(c, requires_grad=True)
    y = bench.torch_fft_circulant(xt, ct, real)
    y.backward(torch.tensor(dy))
    dx, dc = co.circulant_backward_dense(x, c, dy)
    np.testing.assert_allclose(y.detach().numpy(), co.circulant_forward_dense(x, c), atol=1e-12)
    np.testing.assert_allclose(xt.grad.numpy(), dx, atol=1e-12)
    np.testing.assert_allclose(ct.grad.numpy(), dc, atol=1e-12)


@pytest.mark.parametrize("p, nbytes, mflops", [(128, 12_058_624, 501.3), (512, 10_878_976, 220.8),
                                                 (4096, 10_534_912, 170.2)])
def test_circ_algorithmic_counts(p, nbytes, mflops):
    # D=4096, B=256, bf16 activations: five activation passes, three fp32
    # parameter passes; flops count five (I)FFT passes over the activations,
    # three over the parameters and three complex MAC passes
    b, f = bench.circ_algorithmic(256, 4096, p, 2)
    assert b == nbytes
    assert f / 1e6 == pytest.approx(mflops, abs=0.05)


@pytest.mark.parametrize("g0, n, chunk", [(0, 20, 64), (5, 20, 64), (60, 10, 64), (0, 2048, 64), (256, 2048, 64),
                                          (3, 0, 64), (63, 1, 64), (7, 130, 8)])
def test_step_runs_cover_exactly(g0, n, chunk):
    # the timed steps are exactly the requested ones, split only at multiples
    # of the rotation's half (a run's forwards and inverses never share a buffer)
    runs = bench.step_runs(g0, n, chunk)
    assert sum(m for _, m in runs) == n
    g = g0
    for start, m in runs:
        assert start == g and m >= 1
        assert start // chunk == (start + m - 1) // chunk
        g += m


def test_more_than_one_gpu_exits_with_a_message():
    import subprocess
    import sys

    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], capture_output=True, text=True, timeout=300,
                       cwd=os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
    assert r.returncode == 2
    assert "one GPU only" in r.stderr


def test_api_summary_window_and_allocation_count(tmp_path):
    # a fabricated trace: two spin-kernel launches on thread 1, and between
    # them one library launch, a hipMalloc on thread 1 and a hipFree on thread
    # 2 (another thread: outside the window); a hipMalloc before the first spin
    api = [("hipMalloc", 1, 5, 10), ("hipLaunchKernel", 1, 1, 20), ("hipLaunchKernel", 1, 2, 30),
           ("hipMalloc", 1, 6, 35), ("hipFree", 2, 7, 36), ("hipGetLastError", 1, 8, 37),
           ("hipLaunchKernel", 1, 3, 40)]
    ker = {1: "at::cuda::(anonymous namespace)::spin_kernel(long)", 2: "void rdfft::rdfft_fwd_kernel<512>()",
           3: "at::cuda::(anonymous namespace)::spin_kernel(long)"}
    with open(tmp_path / "api_hip_api_trace.csv", "w") as f:
        f.write("Domain,Function,Process_Id,Thread_Id,Correlation_Id,Start_Timestamp,End_Timestamp\n")
        for fn, tid, cid, t in api:
            f.write(f"HIP_RUNTIME_API,{fn},9,{tid},{cid},{t},{t + 1}\n")
    with open(tmp_path / "api_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Correlation_Id,Start_Timestamp,End_Timestamp\n")
        for cid, name in ker.items():
            f.write(f"\"{name}\",{cid},{100 + cid},{110 + cid}\n")
    md = bench.api_summary(str(tmp_path))
    assert "Kernel launches in the window: 1, of which 1 of this library." in md
    assert "Allocation, free or memset calls in the window: 1 (hipMalloc: 1)." in md
    assert "| `hipGetLastError` | 1 |" in md and "hipFree" not in md.split("| HIP function")[1]
