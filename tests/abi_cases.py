"""Host-side argument cases of the C ABI: (entry point, arguments, expected status).

Pointers are plain integers (aligned fake device addresses, never
dereferenced) or None; the stream argument is left out (always NULL).  Every
case either carries an invalid argument or asks for no work, so no call ever
launches a kernel.  test_abi_cpu.py calls them through ctypes on the built
library; test_host_sanitizers_cpu.py runs the same cases through the host
build of the library under AddressSanitizer and UndefinedBehaviorSanitizer.
"""

OK, NULL, SIZE, SHAPE, DTYPE, ALIGN, ALIAS = "OK", "NULL", "SIZE", "SHAPE", "DTYPE", "ALIGN", "ALIAS"
SCRATCH = "SCRATCH"
F32, BF16, F16 = 0, 1, 2
A, B_, C_ = 0x100000, 0x200000, 0x300000
DX, DC = 0x400000, 0x500000
I64_MAX = (1 << 63) - 1


def _rdfft(fn):
    cases = [((None, 4, 512, F32), NULL), ((None, 0, 512, F32), OK), ((A, 0, 4096, BF16), OK)]
    cases += [((A, 4, p, F32), SIZE) for p in (0, 1, 3, 6, 100, 65536, -4)]
    cases += [((A, -1, 512, F32), SIZE), ((A, 1 << 40, 4096, F32), SIZE), ((A, 1 << 26, 32768, F32), SIZE),
              ((A, I64_MAX, 32768, F32), SIZE), ((A, I64_MAX, 2, BF16), SIZE),
              ((A, 4, 512, 3), DTYPE), ((A, 4, 512, -1), DTYPE), ((None, 4, 512, F16), NULL),
              ((0x100004, 4, 512, F32), ALIGN), ((0x100008, 4, 512, BF16), ALIGN)]
    return [(fn, a, e) for a, e in cases]


def _circ_fwd():
    f = "circulant_fwd"
    cases = [
        ((A, C_, B_, 0, 64, 64, 16, F32), OK),
        ((None, C_, B_, 2, 64, 64, 16, F32), NULL),
        ((A, None, B_, 2, 64, 64, 16, F32), NULL),
        ((A, C_, None, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, 2, 64, 64, 12, F32), SIZE),
        ((A, C_, B_, 2, 64, 64, 8192, F32), SIZE),
        ((A, C_, B_, -1, 64, 64, 16, F32), SIZE),
        # activation rows wider than 2^24 features, and a weight grid past 2^40 elements
        ((A, C_, B_, 2, 1 << 25, 64, 16, F32), SIZE),
        ((A, C_, B_, 2, 64, 1 << 25, 16, BF16), SIZE),
        ((A, C_, B_, 2, 1 << 24, 1 << 24, 16, F32), SIZE),
        ((A, C_, B_, I64_MAX, 1 << 24, 1 << 24, 2, F32), SIZE),
        ((A, C_, B_, I64_MAX, 4096, 4096, 4096, BF16), SIZE),
        ((A, C_, B_, 2, I64_MAX - (I64_MAX % 16), 64, 16, F32), SIZE),
        ((A, C_, B_, 2, 60, 64, 16, F32), SHAPE),
        ((A, C_, B_, 2, 64, 72, 16, F32), SHAPE),
        ((A, C_, B_, 2, 0, 64, 16, F32), SHAPE),
        ((A, C_, B_, 2, -64, 64, 16, F32), SHAPE),
        ((A, C_, B_, 2, 64, 64, 16, 9), DTYPE),
        ((0x100002, C_, B_, 2, 64, 64, 16, BF16), ALIGN),
        # y overlapping x or c (c is 4 x 4 x 16 fp32 = 1024 B)
        ((A, C_, 0x100000 + 256, 2, 64, 64, 16, F32), ALIAS),
        ((A, C_, 0x300000 + 1008, 2, 64, 64, 16, F32), ALIAS),
    ]
    return [(f, a, e) for a, e in cases]


def _circ_bwd():
    f = "circulant_bwd"
    cases = [
        ((A, C_, B_, None, None, 2, 64, 64, 16, F32), NULL),  # nothing to compute
        ((None, C_, B_, DX, DC, 2, 64, 64, 16, F32), NULL),
        ((A, C_, None, DX, DC, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, DX, None, 0, 64, 64, 16, F32), OK),  # empty batch, no dc to zero
        ((A, C_, B_, DX, DC, 2, 64, 48, 32, F32), SHAPE),
        ((A, C_, B_, DX, DC, 2, 64, 64, 5, F32), SIZE),
        ((A, C_, B_, DX, DC, 2, 1 << 25, 64, 16, F32), SIZE),
        ((A, C_, B_, DX, DC, I64_MAX, 4096, 4096, 16, F32), SIZE),
        ((A, C_, B_, DX, DC, 2, 64, 64, 16, 3), DTYPE),
        ((A, C_, B_, 0x400004, DC, 2, 64, 64, 16, F32), ALIGN),
        ((A, C_, B_, DX, 0x500004, 0, 64, 64, 16, F32), ALIGN),
        # dx overlapping dy, dc overlapping c / x
        ((A, C_, B_, 0x200000 + 64, DC, 2, 64, 64, 16, F32), ALIAS),
        ((A, C_, B_, DX, 0x300000 + 16, 2, 64, 64, 16, F32), ALIAS),
        ((A, C_, B_, None, 0x100000, 2, 64, 64, 16, F32), ALIAS),
    ]
    return [(f, a, e) for a, e in cases]


def _circ_fwd_zero():
    # the argument checks of circulant_fwd, plus dc (4 x 4 x 16 fp32 = 1024 B);
    # an empty batch still clears dc, so it would launch: not listed
    f = "circulant_fwd_zero"
    cases = [
        ((A, C_, B_, None, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, None, 0, 64, 64, 16, F32), NULL),
        ((None, C_, B_, DC, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, DC, 2, 64, 64, 12, F32), SIZE),
        ((A, C_, B_, DC, 2, 64, 72, 16, F32), SHAPE),
        ((A, C_, B_, DC, 2, 64, 64, 16, 4), DTYPE),
        ((A, C_, B_, 0x500008, 2, 64, 64, 16, F32), ALIGN),
        ((A, C_, B_, 0x500008, 0, 64, 64, 16, F32), ALIGN),
        ((A, C_, B_, 0x300000 + 512, 2, 64, 64, 16, F32), ALIAS),
        ((A, C_, B_, 0x200000 - 512, 2, 64, 64, 16, BF16), ALIAS),
        ((A, C_, B_, 0x100000 + 16, 2, 64, 64, 16, F32), ALIAS),
    ]
    return [(f, a, e) for a, e in cases]


def _circ_bwd_acc():
    # the checks of circulant_bwd; an empty batch adds nothing and launches nothing
    f = "circulant_bwd_acc"
    cases = [
        ((A, C_, B_, None, None, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, DX, DC, 0, 64, 64, 16, F32), OK),
        ((A, C_, B_, None, DC, 0, 64, 64, 16, BF16), OK),
        ((A, None, B_, DX, DC, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, DX, DC, 2, 64, 64, 8192, F32), SIZE),
        ((A, C_, B_, DX, DC, 2, 48, 64, 32, F32), SHAPE),
        ((A, C_, B_, DX, DC, 2, 64, 64, 16, -2), DTYPE),
        ((A, C_, B_, DX, 0x500004, 2, 64, 64, 16, F32), ALIGN),
        ((A, C_, B_, DX, 0x300000 + 1008, 2, 64, 64, 16, F32), ALIAS),
        ((A, C_, B_, 0x500000 - 64, DC, 2, 64, 64, 16, F32), ALIAS),
    ]
    return [(f, a, e) for a, e in cases]


def _circ_bwd_det():
    # circulant_bwd's checks, then dc required and the workspace: 2 tokens of
    # 64 features at p = 16 need one slice of 4 x 4 x 16 floats (1 KiB) per
    # token range; an empty batch needs none (and would launch: not listed)
    f = "circulant_bwd_det"
    WS = 0x600000
    cases = [
        ((A, C_, B_, DX, None, WS, 1 << 20, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, None, None, WS, 1 << 20, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, DX, DC, None, 1 << 20, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, DX, DC, WS, 0, 2, 64, 64, 16, F32), SIZE),
        ((A, C_, B_, DX, DC, WS, -16, 2, 64, 64, 16, F32), SIZE),
        ((A, C_, B_, DX, DC, WS, 1 << 20, 2, 64, 64, 12, F32), SIZE),
        ((A, C_, B_, DX, DC, WS, 1 << 20, 2, 64, 48, 32, F32), SHAPE),
        ((A, C_, B_, DX, DC, WS, 1 << 20, 2, 64, 64, 16, 7), DTYPE),
        ((A, C_, B_, DX, DC, 0x600004, 1 << 20, 2, 64, 64, 16, F32), ALIGN),
        ((A, C_, B_, DX, DC, 0x500000 + 512, 1 << 20, 2, 64, 64, 16, F32), ALIAS),
        ((A, C_, B_, DX, DC, 0x100000 - 256, 1 << 20, 2, 64, 64, 16, BF16), ALIAS),
    ]
    return [(f, a, e) for a, e in cases]


def _circ_bwd_det_noalloc():
    # circulant_bwd's checks, dc required, and the 32 MiB limit of the
    # library's own workspace: at p = 16, 65536 x 65536 features the dc slices
    # alone need 1 GiB (buffers 1 TiB apart so that none overlaps another)
    f = "circulant_bwd_det_noalloc"
    T = 1 << 40
    cases = [
        ((A, C_, B_, DX, None, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, None, None, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, DX, DC, 2, 64, 64, 12, F32), SIZE),
        ((A, C_, B_, DX, DC, 2, 64, 64, 16, 5), DTYPE),
        ((A, C_, B_, DX, 0x500004, 2, 64, 64, 16, F32), ALIGN),
        ((A, C_, B_, DX, 0x300000 + 16, 2, 64, 64, 16, F32), ALIAS),
        ((T, 2 * T, 3 * T, 4 * T, 5 * T, 256, 65536, 65536, 16, F32), SCRATCH),
        ((T, 2 * T, 3 * T, None, 5 * T, 256, 65536, 65536, 16, BF16), SCRATCH),
    ]
    return [(f, a, e) for a, e in cases]


def _det_workspace():
    # the size query of circulant_bwd_det (its last argument is the output
    # pointer); only failing cases, which write nothing through it
    f = "circulant_bwd_det_workspace"
    cases = [
        ((2, 64, 64, 16, 1, None), NULL),
        ((2, 64, 64, 12, 1, B_), SIZE),
        ((2, 64, 64, 8192, 0, B_), SIZE),
        ((-1, 64, 64, 16, 1, B_), SIZE),
        ((2, 60, 64, 16, 1, B_), SHAPE),
        ((I64_MAX, 4096, 4096, 4096, 1, B_), SIZE),
    ]
    return [(f, a, e) for a, e in cases]


def _weight_spectra():
    # c and cs are 4 x 4 x 16 fp32 (1 KiB); every valid call would launch, so
    # only failing ones; 65536 x 65536 features at p = 2 make cs 8 GiB, past
    # the 2 GiB of one buffer resource
    f = "circulant_weight_spectra"
    T = 1 << 40
    cases = [
        ((None, B_, 64, 64, 16), NULL),
        ((C_, None, 64, 64, 16), NULL),
        ((C_, B_, 64, 64, 12), SIZE),
        ((C_, B_, 64, 64, 8192), SIZE),
        ((C_, B_, 60, 64, 16), SHAPE),
        ((C_, B_, 64, 0, 16), SHAPE),
        ((C_, 0x200004, 64, 64, 16), ALIGN),
        ((C_, 0x300000 + 512, 64, 64, 16), ALIAS),
        ((T, 2 * T, 65536, 65536, 2), SIZE),
    ]
    return [(f, a, e) for a, e in cases]


def _circ_fwd_spec():
    # circulant_fwd's checks with cs for c, dc optional, and the size limit of
    # the spectra; an empty batch without dc launches nothing
    f = "circulant_fwd_spec"
    T = 1 << 40
    cases = [
        ((A, C_, B_, None, 0, 64, 64, 16, F32), OK),
        ((None, C_, B_, None, 2, 64, 64, 16, F32), NULL),
        ((A, None, B_, DC, 2, 64, 64, 16, BF16), NULL),
        ((A, C_, B_, None, 2, 64, 64, 12, F32), SIZE),
        ((A, C_, B_, DC, 2, 64, 72, 16, F32), SHAPE),
        ((A, C_, B_, None, 2, 64, 64, 16, 3), DTYPE),
        ((A, C_, B_, 0x500008, 2, 64, 64, 16, F32), ALIGN),
        ((A, C_, 0x100000 + 64, None, 2, 64, 64, 16, F32), ALIAS),
        ((A, C_, B_, 0x300000 + 256, 2, 64, 64, 16, F32), ALIAS),
        ((T, 2 * T, 3 * T, None, 2, 65536, 65536, 2, F32), SIZE),
        ((T, 2 * T, 3 * T, 4 * T, 2, 65536, 65536, 2, BF16), SIZE),
    ]
    return [(f, a, e) for a, e in cases]


def _circ_fwd_step():
    # circulant_fwd's checks, dc optional, cs required and separate from every
    # other buffer; an empty batch still writes cs, so it would launch: not listed
    f = "circulant_fwd_step"
    CS, T = 0x600000, 1 << 40
    cases = [
        ((A, C_, B_, DC, None, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, None, None, 0, 64, 64, 16, F32), NULL),
        ((A, None, B_, DC, CS, 0, 64, 64, 16, F32), NULL),
        ((None, C_, B_, DC, CS, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, DC, CS, 2, 64, 64, 12, F32), SIZE),
        ((A, C_, B_, DC, CS, 2, 64, 48, 32, F32), SHAPE),
        ((A, C_, B_, DC, CS, 2, 64, 64, 16, 6), DTYPE),
        ((A, C_, B_, DC, 0x600004, 2, 64, 64, 16, F32), ALIGN),
        ((A, C_, B_, DC, 0x300000 + 512, 2, 64, 64, 16, F32), ALIAS),
        ((A, C_, B_, DC, 0x500000 + 512, 2, 64, 64, 16, F32), ALIAS),
        ((A, C_, B_, None, 0x100000 + 64, 2, 64, 64, 16, BF16), ALIAS),
        ((A, C_, B_, None, 0x200000 + 64, 2, 64, 64, 16, F32), ALIAS),
        ((T, 2 * T, 3 * T, 4 * T, 5 * T, 2, 65536, 65536, 2, F32), SIZE),
    ]
    return [(f, a, e) for a, e in cases]


def _circ_bwd_spec():
    # circulant_bwd's checks with cs for c (the seventh argument is the
    # accumulate flag) and the size limit of the spectra
    f = "circulant_bwd_spec"
    T = 1 << 40
    cases = [
        ((A, C_, B_, None, None, 0, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, DX, DC, 1, 0, 64, 64, 16, F32), OK),
        ((A, C_, B_, DX, None, 0, 0, 64, 64, 16, F32), OK),
        ((A, None, B_, DX, DC, 0, 2, 64, 64, 16, F32), NULL),
        ((A, C_, B_, DX, DC, 1, 2, 64, 64, 5, F32), SIZE),
        ((A, C_, B_, DX, DC, 0, 2, 48, 64, 32, F32), SHAPE),
        ((A, C_, B_, DX, DC, 0, 2, 64, 64, 16, 9), DTYPE),
        ((A, C_, B_, 0x400004, DC, 0, 2, 64, 64, 16, F32), ALIGN),
        ((A, C_, B_, DX, 0x300000 + 16, 1, 2, 64, 64, 16, F32), ALIAS),
        ((A, C_, B_, 0x200000 + 64, DC, 0, 2, 64, 64, 16, F32), ALIAS),
        ((T, 2 * T, 3 * T, 4 * T, 5 * T, 1, 2, 65536, 65536, 2, F32), SIZE),
    ]
    return [(f, a, e) for a, e in cases]


def _spectrum(fn):
    # argument order: (source, destination, ...): packed then spec for unpack, spec then packed for pack
    cases = [((A, B_, 0, 512, F32), OK), ((None, B_, 4, 512, F32), NULL), ((A, None, 4, 512, BF16), NULL)]
    cases += [((A, B_, 4, p, F32), SIZE) for p in (0, 1, 3, 65536)]
    cases += [((A, B_, -2, 512, F32), SIZE), ((A, B_, I64_MAX, 32768, F32), SIZE), ((A, B_, 4, 512, 7), DTYPE),
              ((0x100008, B_, 4, 512, F16), ALIGN), ((A, 0x200004, 4, 512, F32), ALIGN),
              # 4 rows of 512 floats = 8 KiB packed; 4 x 257 x 8 B spectra
              ((A, 0x100000 + 4096, 4, 512, F32), ALIAS), ((0x200000 + 8176, B_, 4, 512, F32), ALIAS)]
    return [(fn, a, e) for a, e in cases]


def _rdfft2d(fn):
    cases = [((None, 0, 64, 64, F32), OK), ((None, 2, 64, 64, F32), NULL)]
    cases += [((A, 2, h, w, F32), SIZE) for h, w in ((3, 64), (64, 3), (8192, 64), (64, 65536), (1, 64), (64, 1))]
    cases += [((A, -1, 64, 64, F32), SIZE), ((A, 1 << 30, 4096, 4096, F32), SIZE),
              ((A, I64_MAX, 4096, 32768, F32), SIZE), ((A, 2, 64, 64, 5), DTYPE), ((0x100002, 2, 64, 64, F16), ALIGN)]
    return [(fn, a, e) for a, e in cases]


CASES = (_rdfft("rdfft_forward") + _rdfft("rdfft_inverse") + _circ_fwd() + _circ_bwd() + _circ_fwd_zero()
         + _circ_bwd_acc() + _circ_bwd_det() + _circ_bwd_det_noalloc() + _det_workspace() + _weight_spectra()
         + _circ_fwd_spec() + _circ_fwd_step() + _circ_bwd_spec() + _spectrum("rdfft_unpack")
         + _spectrum("rdfft_pack") + _rdfft2d("rdfft2d_forward") + _rdfft2d("rdfft2d_inverse"))
