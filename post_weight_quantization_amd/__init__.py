"""KronQ per-linear-layer quantization solver, native on MI355X (gfx950).

The computation lives in libkq.so (HIP kernels behind the C ABI of
include/kq.h). ``api`` is a thin torch binding with the same entry-point
names; ``layer`` chains the entry points for one layer; ``capture`` feeds
the covariance entry point from a torch model's forward and backward hooks.
Importing this
package raises if the library has not been built.
"""
from . import capture, layer  # noqa: F401
from .capture import CovarianceCapture  # noqa: F401
from ._native import KQError, LIB_PATH  # noqa: F401
from .api import (  # noqa: F401
    kq_accumulate_cov,
    kq_allocate_bits,
    kq_apply_quantized,
    kq_apply_quantized_a4,
    kq_apply_quantized_noalloc,
    kq_biip,
    kq_cholesky_inv,
    kq_form_p,
    kq_gptaq_quantize,
    kq_yaqa_quantize,
    kq_layer_objective,
    kq_pack_codes,
    kq_packed_row_words,
    kq_sensitivity,
    kq_set_kernel_events,
    kq_set_gemm_tile,
    kq_workspace_size,
)
