"""ctypes loader for libkq.so (the C ABI declared in include/kq.h).

The library is built in-tree by ``post_weight_quantization_amd.build``. There is
no fallback: if it is missing, importing this module raises.
"""
from __future__ import annotations

import ctypes
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.environ.get("KQ_LIB_PATH") or os.path.join(HERE, "libkq.so")

KQ_OK, KQ_ERR_ARG, KQ_ERR_SHAPE, KQ_ERR_NOT_PD, KQ_ERR_NONFINITE, KQ_ERR_WORKSPACE, KQ_ERR_HIP, \
    KQ_ERR_UNSUPPORTED = range(8)
STATUS_NAMES = {0: "KQ_OK", 1: "KQ_ERR_ARG", 2: "KQ_ERR_SHAPE", 3: "KQ_ERR_NOT_PD",
                4: "KQ_ERR_NONFINITE", 5: "KQ_ERR_WORKSPACE", 6: "KQ_ERR_HIP", 7: "KQ_ERR_UNSUPPORTED"}
KQ_BF16, KQ_F32 = 0, 1
KQ_NOALLOC_SCRATCH_BYTES = 64 << 20  # include/kq.h
(KQ_OP_ACCUMULATE_COV, KQ_OP_BIIP, KQ_OP_SENSITIVITY, KQ_OP_CHOLESKY_INV, KQ_OP_FORM_P,
 KQ_OP_GPTAQ_QUANTIZE, KQ_OP_LAYER_OBJECTIVE, KQ_OP_APPLY_QUANTIZED,
 KQ_OP_YAQA_QUANTIZE, KQ_OP_APPLY_QUANTIZED_A4) = range(10)

# every symbol include/kq.h declares
EXPORTS = ("kq_last_error", "kq_version", "kq_workspace_size", "kq_accumulate_cov", "kq_biip",
           "kq_sensitivity", "kq_cholesky_inv", "kq_form_p", "kq_gptaq_quantize",
           "kq_allocate_bits", "kq_layer_objective", "kq_set_kernel_events",
           "kq_packed_row_words", "kq_pack_codes", "kq_apply_quantized", "kq_yaqa_quantize",
           "kq_apply_quantized_a4", "kq_apply_quantized_noalloc", "kq_set_gemm_tile")


class kq_quant_cfg(ctypes.Structure):
    _fields_ = [("bits", ctypes.c_int32), ("group", ctypes.c_int32), ("block", ctypes.c_int32),
                ("flags", ctypes.c_int32)]


class KQError(RuntimeError):
    def __init__(self, status: int, message: str, info: int = 0):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status
        self.info = info


if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is not built; run `python post_weight_quantization_amd/build.py`")

lib = ctypes.CDLL(LIB_PATH)

_p = ctypes.c_void_p
_i64 = ctypes.c_int64
_sz = ctypes.c_size_t
_st = ctypes.c_int


def _sig(name, restype, *argtypes):
    f = getattr(lib, name)
    f.restype = restype
    f.argtypes = list(argtypes)
    return f


_sig("kq_last_error", ctypes.c_char_p)
_sig("kq_version", ctypes.c_char_p)
_sig("kq_workspace_size", _st, ctypes.c_int, _i64, _i64, _i64, ctypes.c_int,
     ctypes.POINTER(kq_quant_cfg), ctypes.POINTER(_sz))
_sig("kq_accumulate_cov", _st, _p, _p, _p, ctypes.c_int, _i64, _i64, _i64, ctypes.c_float,
     ctypes.c_float, _p, _p, _p, _p, _sz, _p)
_sig("kq_biip", _st, _p, _p, _p, _p, _i64, _i64, _p, _p, _i64, _i64, _p, _p, _p, _sz, _p)
_sig("kq_sensitivity", _st, _p, _p, _i64, _i64, ctypes.POINTER(ctypes.c_double),
     ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double), _p, _sz, _p)
_sig("kq_cholesky_inv", _st, _p, _i64, ctypes.c_float, _p, ctypes.POINTER(ctypes.c_int32), _p, _sz, _p)
_sig("kq_form_p", _st, _p, _p, _i64, _p, _p, _sz, _p)
_sig("kq_gptaq_quantize", _st, _p, _p, _p, _i64, _i64, ctypes.POINTER(kq_quant_cfg), _p, _p, _p,
     _p, _sz, _p)
_sig("kq_yaqa_quantize", _st, _p, _p, _p, _p, _i64, _i64, ctypes.POINTER(kq_quant_cfg), _p, _p,
     _p, _p, _sz, _p)
_sig("kq_allocate_bits", _st, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64),
     ctypes.c_int32, ctypes.POINTER(ctypes.c_int32), ctypes.c_int32, ctypes.c_double,
     ctypes.POINTER(ctypes.c_int32))
_sig("kq_layer_objective", _st, _p, _p, _p, _p, _p, _i64, _i64, ctypes.POINTER(ctypes.c_double),
     _p, _sz, _p)


_sig("kq_set_kernel_events", _st, ctypes.c_int, _p, _p)
_sig("kq_set_gemm_tile", _st, ctypes.c_int)
_sig("kq_packed_row_words", _st, _i64, ctypes.c_int32, ctypes.POINTER(ctypes.c_int64))
_sig("kq_pack_codes", _st, _p, _i64, _i64, ctypes.c_int32, _p, _p)
_sig("kq_apply_quantized", _st, _p, ctypes.c_int32, _p, _p, ctypes.c_int32, _p, _p, _p, _p, _i64, _i64,
     _p, _i64, _i64, _i64, _p, _p, _sz, _p)
_sig("kq_apply_quantized_noalloc", _st, _p, ctypes.c_int32, _p, _p, ctypes.c_int32, _p, _p, _p, _p, _i64,
     _i64, _p, _i64, _i64, _i64, _p, _p)
_sig("kq_apply_quantized_a4", _st, _p, _p, _p, _p, _p, _p, _p, _i64, _i64, _p, _i64, _i64, _i64,
     ctypes.c_float, _p, _p, _p, _p, _sz, _p)


def check(status: int, info: int = 0) -> None:
    if status != KQ_OK:
        raise KQError(status, lib.kq_last_error().decode(), info)
