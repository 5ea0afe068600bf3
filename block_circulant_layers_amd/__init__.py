"""MI355X-native in-place packed real FFT (rdFFT) and block-circulant layers.

The compute path is the HIP library ``lib/librdfft.so`` (C ABI in
``include/rdfft.h``); :mod:`block_circulant_layers_amd.binding` is its thin
Python binding.  Build with ``python -m block_circulant_layers_amd.build``.
"""

from .binding import (  # noqa: F401
    RDFFT_BF16,
    RDFFT_F16,
    RDFFT_F32,
    RdfftError,
    circulant_bwd,
    circulant_bwd_acc,
    circulant_bwd_det,
    circulant_bwd_det_noalloc,
    circulant_bwd_det_workspace,
    circulant_bwd_spec,
    circulant_fwd,
    circulant_fwd_spec,
    circulant_fwd_step,
    circulant_fwd_zero,
    circulant_weight_spectra,
    lib,
    lib_path,
    rdfft2d_forward,
    rdfft2d_inverse,
    rdfft_forward,
    rdfft_inverse,
    rdfft_pack,
    rdfft_unpack,
)
from .layer import BlockCirculantFunction, BlockCirculantLinear  # noqa: F401
