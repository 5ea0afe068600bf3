"""LDS bank model of the exchange layouts (CPU only).

tests/lds_check/bank_model.cpp lists, thread by thread, the LDS addresses of
every exchange access of the pass schedule for each row length the kernels
instantiate -- through the layout functions of rdfft_device.hpp themselves
(padding, item order) -- and the load loop of the 2D column tiles.  It counts
the extra cycles of each wavefront access in two 32-lane halves over 32 banks,
the count that rocprofv3's SQ_LDS_BANK_CONFLICT reports (exactly, for the
layouts measured: the long rows and the 4096-row column tiles).

The expected figures below are the layouts as chosen: conflict-free except
for pass 16's exchange at 256 <= p <= 2048 (a residue no padding removes: the
first scatter needs an odd stride, this gather one of 4 mod 8) and pass 1024
at p = 16384 (its conflict-free item order measured slower).  A change of any
layout shows up here as a changed count.  The exchanges are the radix-2 stage
groups of Paper-Notes, "四元素对称群 (Proposition 1)", as the kernels pass
them between threads.
"""

from __future__ import annotations

import subprocess

import pytest

from tests.lds_check import build_emu

# extra cycles per row, forward and inverse
ROW = {32: 0, 64: 0, 128: 0, 256: 8, 512: 16, 1024: 32, 2048: 64, 4096: 0, 8192: 0, 16384: 1024, 32768: 0}


@pytest.fixture(scope="module")
def lines():
    exe = build_emu.build("bank")
    out = subprocess.run([exe], capture_output=True, text=True, timeout=300, check=True).stdout
    return [ln.split() for ln in out.splitlines()]


def test_row_exchanges(lines):
    got = {int(f[1]): (int(f[2]), float(f[3]), float(f[4])) for f in lines if f[0] == "row"}
    assert sorted(got) == sorted(ROW)
    for p, want in ROW.items():
        e, fwd, inv = got[p]
        assert e == (32 if p == 32768 else 16)
        assert (fwd, inv) == (want, want), (p, fwd, inv)


def test_column_tiles(lines):
    cols = [f for f in lines if f[0] == "col"]
    assert len(cols) == 8
    for _, h, cl, cs, extra in cols:
        assert int(extra) == 0, (h, cl, cs)
        assert int(cl) * int(cs) * 4 <= 144 * 1024
