"""C-ABI checks that need no GPU: the library loads, exports what include/rdfft.h
declares, and rejects bad arguments on the host before touching any device
memory (the pointers used here are never dereferenced: every call below carries at
least one invalid argument, so no kernel is ever enqueued)."""

import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rdfft.h")

bcl = pytest.importorskip("block_circulant_layers_amd")


def _header_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", src, flags=re.M)))


def _header_defines():
    out = {}
    for name, val in re.findall(r"#define\s+(RDFFT_\w+)\s+(\d+)", open(HEADER).read()):
        out[name] = int(val)
    return out


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(bcl.lib_path()):
        pytest.fail("librdfft.so is not built: run python -m block_circulant_layers_amd.build")
    return bcl.lib()


def test_exports_every_declared_symbol(L):
    names = _header_functions()
    assert set(names) == {"rdfft_abi_version", "rdfft_status_string", "rdfft_forward", "rdfft_inverse",
                          "circulant_fwd", "circulant_bwd", "rdfft_unpack", "rdfft_pack",
                          "rdfft2d_forward", "rdfft2d_inverse"}
    for n in names:
        assert hasattr(L, n), n
    # the binding's signature table covers exactly the header
    assert set(bcl.binding.SIGNATURES) == set(names)


def test_abi_version_and_status_strings(L):
    d = _header_defines()
    assert L.rdfft_abi_version() == d["RDFFT_ABI_VERSION"]
    codes = [v for k, v in d.items() if k.startswith("RDFFT_ERR_") or k == "RDFFT_OK"]
    msgs = {L.rdfft_status_string(c).decode() for c in codes}
    assert len(msgs) == len(codes)  # one distinct message per status
    assert L.rdfft_status_string(12345) == b"unknown status"


D = _header_defines()
OK, NULL, SIZE, SHAPE, DTYPE, ALIGN, ALIAS = (D["RDFFT_OK"], D["RDFFT_ERR_NULL"], D["RDFFT_ERR_SIZE"],
                                              D["RDFFT_ERR_SHAPE"], D["RDFFT_ERR_DTYPE"], D["RDFFT_ERR_ALIGN"],
                                              D["RDFFT_ERR_ALIAS"])
F32, BF16, F16 = D["RDFFT_F32"], D["RDFFT_BF16"], D["RDFFT_F16"]
A = ctypes.c_void_p(0x100000)  # aligned fake device addresses, never dereferenced
B_ = ctypes.c_void_p(0x200000)
C_ = ctypes.c_void_p(0x300000)


@pytest.mark.parametrize("fn", ["rdfft_forward", "rdfft_inverse"])
def test_rdfft_validation(L, fn):
    f = getattr(L, fn)
    assert f(None, 4, 512, F32, None) == NULL
    assert f(None, 0, 512, F32, None) == OK  # empty batch: no-op, pointer unchecked
    assert f(A, 0, 4096, BF16, None) == OK
    for p in (0, 1, 3, 6, 100, 65536, -4):
        assert f(A, 4, p, F32, None) == SIZE, p
    assert f(A, -1, 512, F32, None) == SIZE
    assert f(A, 1 << 40, 4096, F32, None) == SIZE  # element count too large
    assert f(A, 1 << 26, 32768, F32, None) == SIZE
    assert f(A, 4, 512, 3, None) == DTYPE
    assert f(A, 4, 512, -1, None) == DTYPE
    assert f(None, 4, 512, F16, None) == NULL
    assert f(ctypes.c_void_p(0x100004), 4, 512, F32, None) == ALIGN
    assert f(ctypes.c_void_p(0x100008), 4, 512, BF16, None) == ALIGN


def test_circulant_fwd_validation(L):
    f = L.circulant_fwd
    assert f(A, C_, B_, 0, 64, 64, 16, F32, None) == OK  # empty batch
    assert f(None, C_, B_, 2, 64, 64, 16, F32, None) == NULL
    assert f(A, None, B_, 2, 64, 64, 16, F32, None) == NULL
    assert f(A, C_, None, 2, 64, 64, 16, F32, None) == NULL
    assert f(A, C_, B_, 2, 64, 64, 12, F32, None) == SIZE
    assert f(A, C_, B_, 2, 64, 64, 8192, F32, None) == SIZE
    assert f(A, C_, B_, -1, 64, 64, 16, F32, None) == SIZE
    # activation rows wider than 2^24 features, and a weight grid past 2^40 elements
    assert f(A, C_, B_, 2, 1 << 25, 64, 16, F32, None) == SIZE
    assert f(A, C_, B_, 2, 64, 1 << 25, 16, BF16, None) == SIZE
    assert f(A, C_, B_, 2, 1 << 24, 1 << 24, 16, F32, None) == SIZE
    assert f(A, C_, B_, 2, 60, 64, 16, F32, None) == SHAPE
    assert f(A, C_, B_, 2, 64, 72, 16, F32, None) == SHAPE
    assert f(A, C_, B_, 2, 0, 64, 16, F32, None) == SHAPE
    assert f(A, C_, B_, 2, 64, 64, 16, 9, None) == DTYPE
    assert f(ctypes.c_void_p(0x100002), C_, B_, 2, 64, 64, 16, BF16, None) == ALIGN
    # y overlapping x or c
    assert f(A, C_, ctypes.c_void_p(0x100000 + 256), 2, 64, 64, 16, F32, None) == ALIAS
    assert f(A, C_, ctypes.c_void_p(0x300000 + 1008), 2, 64, 64, 16, F32, None) == ALIAS  # c is 1024 B


def test_circulant_bwd_validation(L):
    f = L.circulant_bwd
    DX = ctypes.c_void_p(0x400000)
    DC = ctypes.c_void_p(0x500000)
    assert f(A, C_, B_, None, None, 2, 64, 64, 16, F32, None) == NULL  # nothing to compute
    assert f(None, C_, B_, DX, DC, 2, 64, 64, 16, F32, None) == NULL
    assert f(A, C_, None, DX, DC, 2, 64, 64, 16, F32, None) == NULL
    assert f(A, C_, B_, DX, None, 0, 64, 64, 16, F32, None) == OK  # empty batch, no dc to zero
    assert f(A, C_, B_, DX, DC, 2, 64, 48, 32, F32, None) == SHAPE
    assert f(A, C_, B_, DX, DC, 2, 64, 64, 5, F32, None) == SIZE
    assert f(A, C_, B_, DX, DC, 2, 1 << 25, 64, 16, F32, None) == SIZE
    assert f(A, C_, B_, DX, DC, 2, 64, 64, 16, 3, None) == DTYPE
    assert f(A, C_, B_, ctypes.c_void_p(0x400004), DC, 2, 64, 64, 16, F32, None) == ALIGN
    # dx overlapping dy, dc overlapping c / x
    assert f(A, C_, B_, ctypes.c_void_p(0x200000 + 64), DC, 2, 64, 64, 16, F32, None) == ALIAS
    assert f(A, C_, B_, DX, ctypes.c_void_p(0x300000 + 16), 2, 64, 64, 16, F32, None) == ALIAS
    assert f(A, C_, B_, None, ctypes.c_void_p(0x100000), 2, 64, 64, 16, F32, None) == ALIAS


@pytest.mark.parametrize("fn", ["rdfft_unpack", "rdfft_pack"])
def test_spectrum_validation(L, fn):
    f = getattr(L, fn)
    # argument order: (source, destination, ...) -- packed then spec for unpack, spec then packed for pack
    assert f(A, B_, 0, 512, F32, None) == OK  # empty: no-op
    assert f(None, B_, 4, 512, F32, None) == NULL
    assert f(A, None, 4, 512, BF16, None) == NULL
    for p in (0, 1, 3, 65536):
        assert f(A, B_, 4, p, F32, None) == SIZE, p
    assert f(A, B_, -2, 512, F32, None) == SIZE
    assert f(A, B_, 4, 512, 7, None) == DTYPE
    assert f(ctypes.c_void_p(0x100008), B_, 4, 512, F16, None) == ALIGN
    assert f(A, ctypes.c_void_p(0x200004), 4, 512, F32, None) == ALIGN
    # 4 rows of 512 floats = 8 KiB packed; 4 x 257 x 8 B spectra
    assert f(A, ctypes.c_void_p(0x100000 + 4096), 4, 512, F32, None) == ALIAS
    assert f(ctypes.c_void_p(0x200000 + 8176), B_, 4, 512, F32, None) == ALIAS


@pytest.mark.parametrize("fn", ["rdfft2d_forward", "rdfft2d_inverse"])
def test_rdfft2d_validation(L, fn):
    f = getattr(L, fn)
    assert f(None, 0, 64, 64, F32, None) == OK  # no arrays: no-op
    assert f(None, 2, 64, 64, F32, None) == NULL
    for h, w in ((3, 64), (64, 3), (8192, 64), (64, 65536), (1, 64), (64, 1)):
        assert f(A, 2, h, w, F32, None) == SIZE, (h, w)
    assert f(A, -1, 64, 64, F32, None) == SIZE
    assert f(A, 1 << 30, 4096, 4096, F32, None) == SIZE
    assert f(A, 2, 64, 64, 5, None) == DTYPE
    assert f(ctypes.c_void_p(0x100002), 2, 64, 64, F16, None) == ALIGN


def test_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(4, 16)
    with pytest.raises(ValueError):
        bcl.rdfft_forward(x)
    with pytest.raises(ValueError):
        bcl.circulant_fwd(x, torch.zeros(1, 1, 16))
