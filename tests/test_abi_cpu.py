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

from tests import abi_cases  # noqa: E402

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
                          "circulant_fwd", "circulant_bwd", "circulant_fwd_zero", "circulant_bwd_acc",
                          "circulant_bwd_det", "circulant_bwd_det_workspace", "circulant_bwd_det_noalloc",
                          "circulant_weight_spectra", "circulant_fwd_step", "circulant_fwd_spec", "circulant_bwd_spec",
                          "rdfft_unpack", "rdfft_pack",
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
STATUS = {"OK": D["RDFFT_OK"], "NULL": D["RDFFT_ERR_NULL"], "SIZE": D["RDFFT_ERR_SIZE"],
          "SHAPE": D["RDFFT_ERR_SHAPE"], "DTYPE": D["RDFFT_ERR_DTYPE"], "ALIGN": D["RDFFT_ERR_ALIGN"],
          "ALIAS": D["RDFFT_ERR_ALIAS"], "SCRATCH": D["RDFFT_ERR_SCRATCH"]}


def test_case_constants_match_header():
    assert (abi_cases.F32, abi_cases.BF16, abi_cases.F16) == (D["RDFFT_F32"], D["RDFFT_BF16"], D["RDFFT_F16"])


@pytest.mark.parametrize("fn,args,want", abi_cases.CASES,
                         ids=[f"{c[0]}-{i}" for i, c in enumerate(abi_cases.CASES)])
def test_validation(L, fn, args, want):
    f = getattr(L, fn)
    # pointer positions: the leading arguments (and, for the workspace query,
    # its last one); circulant_bwd_det's seventh is the workspace size
    n_ptr = {"rdfft_forward": 1, "rdfft_inverse": 1, "circulant_fwd": 3, "circulant_bwd": 5,
             "circulant_fwd_zero": 4, "circulant_bwd_acc": 5, "circulant_bwd_det": 6,
             "circulant_bwd_det_workspace": 0, "circulant_bwd_det_noalloc": 5, "circulant_weight_spectra": 2,
             "circulant_fwd_spec": 4, "circulant_fwd_step": 5, "circulant_bwd_spec": 5, "rdfft_unpack": 2,
             "rdfft_pack": 2, "rdfft2d_forward": 1, "rdfft2d_inverse": 1}[fn]
    ptrs = set(range(n_ptr)) | ({len(args) - 1} if fn == "circulant_bwd_det_workspace" else set())
    cargs = [(ctypes.c_void_p(a) if a is not None else None) if i in ptrs else a for i, a in enumerate(args)]
    if fn == "circulant_bwd_det_workspace":  # an int64_t* output, no stream argument
        out = args[-1]
        cargs[-1] = ctypes.cast(out, ctypes.POINTER(ctypes.c_int64)) if out is not None else None
        assert f(*cargs) == STATUS[want]
    else:
        assert f(*cargs, None) == STATUS[want]


def test_layer_options_that_do_not_combine():
    with pytest.raises(ValueError):
        bcl.BlockCirculantLinear(64, 64, 16, device="cpu", weight_spectra=True, deterministic=True)


def test_binding_refuses_cpu_tensors():
    import torch

    x = torch.zeros(4, 16)
    with pytest.raises(ValueError):
        bcl.rdfft_forward(x)
    with pytest.raises(ValueError):
        bcl.circulant_fwd(x, torch.zeros(1, 1, 16))
