"""Host-side checks of bench.py's helpers (no GPU).

The torch.fft forms that bench.py times beside the layer as context must be
the same linear map as the block-circulant layer (Paper-Notes, "循环矩阵训练
适配"): checked here against the oracle's dense forward and backward in float64.
"""
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
