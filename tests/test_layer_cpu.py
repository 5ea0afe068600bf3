"""Host-side behaviour of the autograd layer: construction and loud failure
without a GPU (there is no CPU path)."""

import math

import pytest
import torch

import block_circulant_layers_amd as bcl


def test_parameter_shape_and_init():
    g = torch.Generator().manual_seed(5)
    layer = bcl.BlockCirculantLinear(4096, 2048, 128, generator=g)
    assert tuple(layer.c.shape) == (16, 32, 128) and layer.c.dtype == torch.float32
    std = float(layer.c.detach().std())
    assert abs(std * math.sqrt(4096) - 1) < 0.01
    assert "p=128" in repr(layer)


@pytest.mark.parametrize("d_in,d_out,p", [(64, 64, 3), (64, 64, 48), (60, 64, 16), (64, 60, 16), (64, 64, 1)])
def test_rejects_bad_block_size(d_in, d_out, p):
    with pytest.raises(ValueError):
        bcl.BlockCirculantLinear(d_in, d_out, p)


def test_cpu_tensors_fail_loudly():
    layer = bcl.BlockCirculantLinear(64, 64, 16)
    with pytest.raises((ValueError, RuntimeError)):
        layer(torch.zeros(2, 64))
