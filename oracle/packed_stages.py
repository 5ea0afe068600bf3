"""The pages' in-place packed Cooley-Tukey, in plain Python -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this module.  It shares no code with the HIP library.

This is the method itself, step by step in the pages' order, for small rows:
it exists to pin our reading of the pages (which index groups a stage touches,
how the inverse undoes it) against the plain DFT in ``rdfft_oracle``.

Forward (Paper-Notes page, "整体框架" and "四元素对称群 (Proposition 1)"):
radix-2 decimation in time.  The row is first put in bit-reversed order (the
pages leave the input order open; "first half = transform of the even
samples" is the plain reading of their example and needs it).  Stage m
(m = 2, 4, ..., r) merges, inside every m-block starting at g, the packed
m/2-point spectra E (first half) and O (second half) into the packed m-point
spectrum, in place:

* DC pair (g, g+m/2):           (E_0, O_0) -> (E_0 + O_0, E_0 - O_0);
* quarter pair (m >= 4):        slot g+3m/4 is negated, since
                                y_{m/4} = E_{m/4} - i O_{m/4};
* four-element group, 0<k<m/4:  slots {g+k, g+m/2-k, g+m/2+k, g+m-k} hold
                                (Re E_k, Im E_k, Re O_k, Im O_k); with
                                t = W_m^k O_k and W_m = exp(-2 pi i / m) they
                                receive (Re(E+t), Re(E-t), -Im(E-t), Im(E+t)),
                                i.e. y_k at (g+k, g+m-k) and
                                y_{m/2-k} = conj(E-t) at (g+m/2-k, g+m/2+k).

The pages' example: at m = 16, k = 2 the 8-point pair (2, 6) meets (10, 14)
and the results pair as (2, 14) and (6, 10).

Inverse (Paper-Notes page, "原地 IFFT 设计"): the same butterfly graph run
backwards, m = r, r/2, ..., 2, then the bit reversal undone.  For a group,
E = (y_k + y_{m/2+k}) / 2 and O = (y_k - y_{m/2+k}) / (2 W_m^k), where
y_{m/2+k} = conj(y_{m/2-k}) is read from slots (g+m/2-k, g+m/2+k).  The DC
pair becomes ((a+b)/2, (a-b)/2) and the quarter slot is negated back.
"""

from __future__ import annotations

import cmath

__all__ = [
    "bit_reverse_indices",
    "group_slots",
    "forward_stages",
    "inverse_stages",
]


def _log2(r: int) -> int:
    if r < 2 or r & (r - 1):
        raise ValueError(f"row length must be a power of two >= 2, got {r}")
    return r.bit_length() - 1


def bit_reverse_indices(r: int) -> list[int]:
    """rev[j] = j with its log2(r) bits reversed."""
    n = _log2(r)
    out = []
    for j in range(r):
        v = 0
        for b in range(n):
            if j >> b & 1:
                v |= 1 << (n - 1 - b)
        out.append(v)
    return out


def group_slots(g: int, m: int, k: int) -> tuple[int, int, int, int]:
    """Slots of the four-element group of stage m, block start g, 0 < k < m/4."""
    if not 0 < k < m // 4:
        raise ValueError("group index k must satisfy 0 < k < m/4")
    h = m // 2
    return (g + k, g + h - k, g + h + k, g + m - k)


def _twiddle(m: int, k: int) -> complex:
    return cmath.exp(-2j * cmath.pi * k / m)


def forward_stages(x: list[float], last_stage: int | None = None) -> list[float]:
    """Packed forward transform of one real row by the pages' stages (float64).

    ``last_stage`` stops after stage m = last_stage (default: r), leaving every
    last_stage-block holding the packed spectrum of its decimated subsequence.
    """
    r = len(x)
    _log2(r)
    stop = r if last_stage is None else last_stage
    rev = bit_reverse_indices(r)
    a = [float(x[rev[j]]) for j in range(r)]
    m = 2
    while m <= stop:
        h = m // 2
        for g in range(0, r, m):
            e0, o0 = a[g], a[g + h]
            a[g], a[g + h] = e0 + o0, e0 - o0
            if m >= 4:
                a[g + 3 * m // 4] = -a[g + 3 * m // 4]
            for k in range(1, m // 4):
                s1, s2, s3, s4 = group_slots(g, m, k)
                e = complex(a[s1], a[s2])
                o = complex(a[s3], a[s4])
                t = _twiddle(m, k) * o
                p, q = e + t, e - t
                a[s1], a[s2], a[s3], a[s4] = p.real, q.real, -q.imag, p.imag
        m *= 2
    return a


def inverse_stages(z: list[float]) -> list[float]:
    """Inverse of :func:`forward_stages`, with the 1/2 of every stage (float64)."""
    r = len(z)
    _log2(r)
    a = [float(v) for v in z]
    m = r
    while m >= 2:
        h = m // 2
        for g in range(0, r, m):
            for k in range(1, m // 4):
                s1, s2, s3, s4 = group_slots(g, m, k)
                yk = complex(a[s1], a[s4])
                yhk = complex(a[s2], -a[s3])  # y_{m/2+k} = conj(y_{m/2-k})
                e = (yk + yhk) / 2
                o = (yk - yhk) / (2 * _twiddle(m, k))
                a[s1], a[s2], a[s3], a[s4] = e.real, e.imag, o.real, o.imag
            if m >= 4:
                a[g + 3 * m // 4] = -a[g + 3 * m // 4]
            y0, yh = a[g], a[g + h]
            a[g], a[g + h] = (y0 + yh) / 2, (y0 - yh) / 2
        m //= 2
    rev = bit_reverse_indices(r)
    x = [0.0] * r
    for j in range(r):
        x[rev[j]] = a[j]
    return x
