"""circulant_bwd_det_noalloc against circulant_bwd_det, the call it varies.

The allocation-free call takes its workspace from the library's per-GPU array
instead of an argument and must give the same dx and dc, bit for bit, as
circulant_bwd_det on the same inputs (the same kernels sum the same slices in
the same order).  Two calls in a row, the second with a smaller input: the
array still holds the first call's slices, which the second must not read.
The torch allocator must see nothing allocated during the calls, and a shape
whose workspace exceeds the array is refused with RDFFT_ERR_SCRATCH, nothing
written.  Gradients: Paper-Notes page, "循环矩阵训练适配".
"""

import pytest
import torch

import block_circulant_layers_amd as bcl
from block_circulant_layers_amd import synthetic as syn
from tests.gpu_util import device_input

pytestmark = pytest.mark.gpu

RDFFT_ERR_SCRATCH = 8


def _inputs(batch, d_in, d_out, p, dtype, index):
    q, k = d_out // p, d_in // p
    x, _ = device_input((batch, d_in), syn.WL_TEST, syn.T_X, index, dtype=dtype)
    c, _ = device_input((q, k, p), syn.WL_TEST, syn.T_C, index, scale=d_in**-0.5, dtype="f32")
    dy, _ = device_input((batch, d_out), syn.WL_TEST, syn.T_DY, index, dtype=dtype)
    return x, c, dy


def test_noalloc_matches_det_twice():
    # the adapter shape with dx (8 MiB of slices), then a smaller one, dc alone
    # (p = 512, time-domain slices), then small p with spectral slices
    for batch, d_in, d_out, p, dtype, want_dx in ((2048, 4096, 4096, 1024, "bf16", True),
                                                  (96, 2048, 2048, 512, "f32", False),
                                                  (33, 256, 128, 16, "f32", True)):
        print(f"no-alloc det B={batch} d_in={d_in} d_out={d_out} p={p} {dtype} dx={want_dx}", flush=True)
        x, c, dy = _inputs(batch, d_in, d_out, p, dtype, p + 11)
        dx_ref, dc_ref = bcl.circulant_bwd_det(x, c, dy, need_dx=want_dx)
        dx = torch.full_like(x, float("nan")) if want_dx else None
        dc = torch.full_like(c, float("nan"))
        torch.cuda.synchronize()
        before = torch.cuda.memory_allocated()
        bcl.circulant_bwd_det_noalloc(x, c, dy, dx, dc)
        torch.cuda.synchronize()
        assert torch.cuda.memory_allocated() == before
        assert torch.equal(dc, dc_ref)
        if want_dx:
            assert torch.equal(dx, dx_ref)


def test_noalloc_refuses_a_workspace_over_its_array():
    # p = 16, 16384 x 16384, 64 tokens: 64 MiB of slices, twice the array
    batch, d, p = 64, 16384, 16
    assert bcl.circulant_bwd_det_workspace(batch, d, d, p, False) > 32 << 20
    x, c, dy = _inputs(batch, d, d, p, "bf16", 3)
    dc = torch.full_like(c, 5.0)
    with pytest.raises(bcl.RdfftError) as err:
        bcl.circulant_bwd_det_noalloc(x, c, dy, None, dc)
    assert err.value.status == RDFFT_ERR_SCRATCH
    torch.cuda.synchronize()
    assert torch.all(dc == 5.0)
