"""Pins of the fp64 oracle against things other than itself (CPU only).

Each oracle function is checked against at least one of: a brute-force DFT
with exact angle reduction, closed forms derived by hand, the pages' worked
index example, finite differences, and algebraic invariants.  The pins are
chosen so that a dropped term, a wrong sign, a swapped Re/Im slot, a wrong
circulant orientation or a transposed operand fails at least one of them.
"""

import math
import os

import numpy as np
import pytest

from oracle import circulant_oracle as co
from oracle import packed_stages as ps
from oracle import rdfft_oracle as ro

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
POW2 = [2, 4, 8, 16, 32, 64]


def brute_dft(x):
    """y_k = sum_n x_n exp(-2 pi i k n / r), with (k n mod r) reduced before the angle."""
    r = len(x)
    y = np.zeros(r, dtype=np.complex128)
    for k in range(r):
        acc = 0j
        for n in range(r):
            ang = 2.0 * math.pi * ((k * n) % r) / r
            acc += x[n] * complex(math.cos(ang), -math.sin(ang))
        y[k] = acc
    return y


def rng(seed):
    return np.random.default_rng(seed)


# ----------------------------------------------------------------------------
# rdfft_oracle: forward layout against a brute-force DFT
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("r", POW2)
def test_forward_matches_bruteforce_layout(r):
    x = rng(r).standard_normal(r)
    z = ro.rdfft_forward(x[None, :])[0]
    y = brute_dft(x)
    tol = 1e-12 * max(1.0, np.abs(y).max())
    # y_0 and y_{r/2} are real and sit at 0 and r/2
    assert abs(y[0].imag) < tol and abs(y[r // 2].imag) < tol
    assert abs(z[0] - y[0].real) < tol
    assert abs(z[r // 2] - y[r // 2].real) < tol
    for k in range(1, r // 2):
        assert abs(z[k] - y[k].real) < tol, k  # Re y_k at index k
        assert abs(z[r - k] - y[k].imag) < tol, k  # Im y_k at index r-k
        # the other half of the spectrum is the conjugate (nothing lost)
        assert abs(y[r - k] - np.conj(y[k])) < tol


def test_hand_p2_p4():
    x0, x1, x2, x3 = 1.5, -2.0, 0.25, 3.0
    assert np.allclose(ro.rdfft_forward(np.array([[x0, x1]]))[0], [x0 + x1, x0 - x1], atol=1e-14)
    # p = 4 by hand: y1 = (x0 - x2) - i (x1 - x3), y2 = x0 - x1 + x2 - x3
    want = [x0 + x1 + x2 + x3, x0 - x2, x0 - x1 + x2 - x3, -(x1 - x3)]
    assert np.allclose(ro.rdfft_forward(np.array([[x0, x1, x2, x3]]))[0], want, atol=1e-14)


@pytest.mark.parametrize("r", [8, 16, 64, 512, 4096])
def test_closed_forms(r):
    n = np.arange(r)
    zero_but = lambda idx, val: np.where(np.arange(r) == idx, val, 0.0)  # noqa: E731
    # delta_0: every Re slot (0..r/2) = 1, every Im slot = 0
    d = np.zeros(r)
    d[0] = 1.0
    want = np.where(np.arange(r) <= r // 2, 1.0, 0.0)
    assert np.allclose(ro.rdfft_forward(d[None])[0], want, atol=1e-12)
    # constant 1: [0] = r
    assert np.allclose(ro.rdfft_forward(np.ones((1, r)))[0], zero_but(0, r), atol=1e-9)
    # (-1)^n: [r/2] = r
    assert np.allclose(ro.rdfft_forward(((-1.0) ** n)[None])[0], zero_but(r // 2, r), atol=1e-9)
    # cos(2 pi n / r): [1] = r/2 ; sin(2 pi n / r): [r-1] = -r/2 (fixes the exponent sign)
    assert np.allclose(ro.rdfft_forward(np.cos(2 * np.pi * n / r)[None])[0], zero_but(1, r / 2), atol=1e-9)
    assert np.allclose(ro.rdfft_forward(np.sin(2 * np.pi * n / r)[None])[0], zero_but(r - 1, -r / 2), atol=1e-9)
    # cos(2 pi 3 n / r) and sin: bin 3
    assert np.allclose(ro.rdfft_forward(np.cos(6 * np.pi * n / r)[None])[0], zero_but(3, r / 2), atol=1e-9)
    assert np.allclose(ro.rdfft_forward(np.sin(6 * np.pi * n / r)[None])[0], zero_but(r - 3, -r / 2), atol=1e-9)
    # ramp: [0] = r(r-1)/2, [k] = -r/2 (0<k<=r/2), [r-k] = (r/2) cot(pi k / r)
    want = np.empty(r)
    want[0] = r * (r - 1) / 2
    for k in range(1, r // 2 + 1):
        want[k] = -r / 2
    for k in range(1, r // 2):
        want[r - k] = (r / 2) / math.tan(math.pi * k / r)
    got = ro.rdfft_forward(n.astype(float)[None])[0]
    assert np.allclose(got, want, rtol=1e-11, atol=1e-9 * r)


def test_golden_ramp_p8():
    vals = [float(v) for v in open(os.path.join(GOLDEN, "ramp_p8.txt")) if not v.startswith("#") and v.strip()]
    got = ro.rdfft_forward(np.arange(8.0)[None])[0]
    assert np.allclose(got, vals, atol=1e-10)


@pytest.mark.parametrize("r", [2, 4, 16, 128, 4096])
def test_roundtrip_both_ways(r):
    x = rng(1000 + r).standard_normal((3, r))
    assert np.allclose(ro.rdfft_inverse(ro.rdfft_forward(x)), x, atol=1e-12)
    # every packed vector is a valid spectrum: forward(inverse(z)) = z
    z = rng(2000 + r).standard_normal((3, r))
    assert np.allclose(ro.rdfft_forward(ro.rdfft_inverse(z)), z, atol=1e-10)


@pytest.mark.parametrize("r", [4, 32, 1024])
def test_parseval_packed(r):
    x = rng(3000 + r).standard_normal(r)
    z = ro.rdfft_forward(x[None])[0]
    mid = np.ones(r, dtype=bool)
    mid[0] = mid[r // 2] = False
    energy = (z[0] ** 2 + z[r // 2] ** 2 + 2.0 * np.sum(z[mid] ** 2)) / r
    assert abs(energy - np.sum(x**2)) < 1e-10 * np.sum(x**2)


@pytest.mark.parametrize("r,s", [(16, 1), (16, 5), (256, 37)])
def test_shift_theorem(r, s):
    x = rng(4000 + r).standard_normal(r)
    z = ro.rdfft_forward(x[None])[0]
    zs = ro.rdfft_forward(np.roll(x, s)[None])[0]
    # y'_k = y_k * exp(-2 pi i k s / r), written with slots directly
    assert abs(zs[0] - z[0]) < 1e-10
    assert abs(zs[r // 2] - z[r // 2] * (-1) ** s) < 1e-10
    for k in range(1, r // 2):
        th = -2 * math.pi * ((k * s) % r) / r
        re = z[k] * math.cos(th) - z[r - k] * math.sin(th)
        im = z[k] * math.sin(th) + z[r - k] * math.cos(th)
        assert abs(zs[k] - re) < 1e-10 and abs(zs[r - k] - im) < 1e-10


def test_linearity():
    r = 64
    a, b = rng(5).standard_normal((2, r))
    lhs = ro.rdfft_forward((2.5 * a - 0.75 * b)[None])[0]
    rhs = 2.5 * ro.rdfft_forward(a[None])[0] - 0.75 * ro.rdfft_forward(b[None])[0]
    assert np.allclose(lhs, rhs, atol=1e-12)


@pytest.mark.parametrize("r", [2, 4, 16, 64])
def test_packed_product_is_circular_convolution(r):
    a, b = rng(6000 + r).standard_normal((2, r))
    conv = np.array([sum(a[m] * b[(n - m) % r] for m in range(r)) for n in range(r)])
    corr = np.array([sum(a[m] * b[(n + m) % r] for m in range(r)) for n in range(r)])
    fa, fb = ro.rdfft_forward(a[None])[0], ro.rdfft_forward(b[None])[0]
    assert np.allclose(ro.rdfft_inverse(ro.packed_product(fa, fb)[None])[0], conv, atol=1e-11)
    assert np.allclose(ro.rdfft_inverse(ro.packed_product(fa, fb, conj_a=True)[None])[0], corr, atol=1e-11)


def test_rejects_bad_lengths():
    for r in (1, 3, 6, 12):
        with pytest.raises(ValueError):
            ro.rdfft_forward(np.zeros((1, r)))


# ----------------------------------------------------------------------------
# packed_stages: the pages' algorithm, pinned to the DFT and the worked example
# ----------------------------------------------------------------------------


@pytest.mark.parametrize("r", [2, 4, 8, 16, 32, 64, 256])
def test_stages_equal_dft(r):
    x = rng(7000 + r).standard_normal(r)
    z = np.array(ps.forward_stages(list(x)))
    y = brute_dft(x) if r <= 64 else np.fft.fft(x)
    want = np.empty(r)
    want[0], want[r // 2] = y[0].real, y[r // 2].real
    for k in range(1, r // 2):
        want[k], want[r - k] = y[k].real, y[k].imag
    assert np.allclose(z, want, atol=1e-11 * r)


@pytest.mark.parametrize("r", [2, 4, 8, 32, 128])
def test_stages_inverse(r):
    x = rng(8000 + r).standard_normal(r)
    assert np.allclose(ps.inverse_stages(ps.forward_stages(list(x))), x, atol=1e-12)
    z = rng(8100 + r).standard_normal(r)
    assert np.allclose(ps.inverse_stages(list(z)), ro.rdfft_inverse(z[None])[0], atol=1e-12)


def _golden_kv(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        if line.startswith("#") or ":" not in line:
            continue
        k, v = line.split(":", 1)
        out[k.strip()] = [int(t) for t in v.split()]
    return out


def test_proposition1_worked_example():
    g = _golden_kv("prop1_group_m16.txt")
    m, k = g["stage"][0], g["k"][0]
    assert list(ps.group_slots(0, m, k)) == g["group_slots"]
    x = rng(9).standard_normal(16)
    # before stage 16: the first 8-block holds the packed 8-point spectrum of the
    # even samples, the second that of the odd samples (decimation in time)
    mid = ps.forward_stages(list(x), last_stage=8)
    ye, yo = brute_dft(x[0::2]), brute_dft(x[1::2])
    a, b = g["even_pair"]
    assert abs(complex(mid[a], mid[b]) - ye[k]) < 1e-12
    a, b = g["odd_pair"]
    assert abs(complex(mid[a], mid[b]) - yo[k]) < 1e-12
    # after stage 16: (2, 14) holds y_2 and (6, 10) holds y_6
    out = ps.forward_stages(list(x))
    y = brute_dft(x)
    a, b = g["result_pair_a"]
    assert abs(complex(out[a], out[b]) - y[k]) < 1e-12
    a, b = g["result_pair_b"]
    assert abs(complex(out[a], out[b]) - y[m // 2 - k]) < 1e-12


def test_group_slots_partition_each_stage():
    # every stage touches each slot of a block exactly once (in place, no workspace)
    r = 64
    m = 2
    while m <= r:
        seen = []
        for g0 in range(0, r, m):
            seen += [g0, g0 + m // 2]
            if m >= 4:
                seen += [g0 + m // 4, g0 + 3 * m // 4]
            for k in range(1, m // 4):
                seen += list(ps.group_slots(g0, m, k))
        assert sorted(seen) == list(range(r)), m
        m *= 2


# ----------------------------------------------------------------------------
# circulant_oracle
# ----------------------------------------------------------------------------


def test_hand_example_p2():
    # one 2x2 circulant block generated by c = (2, 3): [[2, 3], [3, 2]]
    c = np.array([[[2.0, 3.0]]])
    x = np.array([[5.0, 7.0]])
    assert np.allclose(co.circulant_forward_dense(x, c), [[31.0, 29.0]])
    assert np.allclose(co.circulant_forward_fft(x, c), [[31.0, 29.0]])


def test_weight_special_cases():
    q = k = 3
    p = 8
    c = np.zeros((q, k, p))
    for i in range(q):
        c[i, i, 0] = 1.0
    assert np.allclose(co.block_circulant_weight(c), np.eye(q * p))
    # c = delta_s in one block: (C x)[a] = x[(a - s) mod p], i.e. a cyclic shift
    s = 3
    c = np.zeros((1, 1, p))
    c[0, 0, s] = 1.0
    x = rng(11).standard_normal((2, p))
    assert np.allclose(co.circulant_forward_dense(x, c), np.roll(x, s, axis=1))
    assert np.allclose(co.circulant_forward_fft(x, c), np.roll(x, s, axis=1))
    # the generator is the first column of its block
    c = rng(12).standard_normal((2, 3, p))
    w = co.block_circulant_weight(c)
    for i in range(2):
        for j in range(3):
            assert np.allclose(w[i * p:(i + 1) * p, j * p], c[i, j])


def test_pages_formula_matches_dense_single_block():
    # circ(c) x = IFFT(FFT(c) * FFT(x)) with the packed oracle transforms
    p = 32
    c = rng(13).standard_normal(p)
    x = rng(14).standard_normal(p)
    via_fft = ro.rdfft_inverse(ro.packed_product(ro.rdfft_forward(c[None])[0], ro.rdfft_forward(x[None])[0])[None])[0]
    dense = co.circulant_forward_dense(x[None], c[None, None])[0]
    assert np.allclose(via_fft, dense, atol=1e-12)


SHAPES = [(2, 64, 64, 16), (3, 32, 64, 8), (5, 48, 16, 16), (4, 8, 8, 2), (2, 128, 256, 128)]


@pytest.mark.parametrize("b,din,dout,p", SHAPES)
def test_dense_vs_fft(b, din, dout, p):
    r = rng(b * 1000 + din + dout + p)
    x = r.standard_normal((b, din))
    c = r.standard_normal((dout // p, din // p, p))
    dy = r.standard_normal((b, dout))
    assert np.allclose(co.circulant_forward_dense(x, c), co.circulant_forward_fft(x, c), atol=1e-10)
    dx1, dc1 = co.circulant_backward_dense(x, c, dy)
    dx2, dc2 = co.circulant_backward_fft(x, c, dy)
    assert np.allclose(dx1, dx2, atol=1e-10)
    assert np.allclose(dc1, dc2, atol=1e-10)


def test_finite_differences():
    r = rng(21)
    b, din, dout, p = 2, 8, 12, 4
    x = r.standard_normal((b, din))
    c = r.standard_normal((dout // p, din // p, p))
    dy = r.standard_normal((b, dout))

    def loss(xx, cc):
        return float(np.sum(dy * co.circulant_forward_dense(xx, cc)))

    dx, dc = co.circulant_backward_dense(x, c, dy)
    h = 1e-6
    for idx in np.ndindex(*x.shape):
        e = np.zeros_like(x)
        e[idx] = h
        num = (loss(x + e, c) - loss(x - e, c)) / (2 * h)
        assert abs(num - dx[idx]) < 1e-7
    for idx in np.ndindex(*c.shape):
        e = np.zeros_like(c)
        e[idx] = h
        num = (loss(x, c + e) - loss(x, c - e)) / (2 * h)
        assert abs(num - dc[idx]) < 1e-7


def test_adjoint_identities():
    r = rng(22)
    b, d, p = 6, 64, 16
    x = r.standard_normal((b, d))
    c = r.standard_normal((d // p, d // p, p))
    dy = r.standard_normal((b, d))
    y = co.circulant_forward_fft(x, c)
    dx, dc = co.circulant_backward_fft(x, c, dy)
    s = np.sum(dy * y)
    assert abs(s - np.sum(dx * x)) < 1e-9 * abs(s) + 1e-9
    assert abs(s - np.sum(dc * c)) < 1e-9 * abs(s) + 1e-9
