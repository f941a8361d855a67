"""ctypes loader for libmx.so: argument types only, no logic."""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmx.so")

_c = ctypes


class QuantItem(ctypes.Structure):
    """mx_quant_item of include/mx.h."""
    _fields_ = [("src", _c.c_void_p), ("rows", _c.c_int64), ("cols", _c.c_int64), ("ld", _c.c_int64),
                ("codes", _c.c_void_p), ("scales", _c.c_void_p)]


QUANT_BATCH_MAX = 32   # MX_QUANT_BATCH_MAX
AMAX_WORDS = 256        # MX_AMAX_WORDS
AMAX_MAX_WORDS = 256    # MX_AMAX_MAX_WORDS
SCRATCH_BYTES = 64 << 20   # MX_SCRATCH_BYTES

# every symbol include/mx.h declares, with (restype, argtypes)
SIGNATURES = {
    "mx_version": (_c.c_int, []),
    "mx_k_pad": (_c.c_int64, [_c.c_int64]),
    "mx_codes_bytes": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int, _c.c_int]),
    "mx_scales_bytes": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int, _c.c_int]),
    "mx_quantize": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p, _c.c_void_p,
                               _c.c_int, _c.c_int, _c.c_void_p]),
    "mx_quantize_batch": (_c.c_int, [_c.POINTER(QuantItem), _c.c_int, _c.c_int, _c.c_void_p]),
    "mx_quantize_batch_amax": (_c.c_int, [_c.POINTER(QuantItem), _c.c_int, _c.c_int, _c.c_void_p, _c.c_void_p]),
    "mx_quantize_amax": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p, _c.c_void_p,
                                    _c.c_int, _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p]),
    "mx_layernorm_quantize": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p, _c.c_void_p,
                                         _c.c_float, _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p]),
    "mx_quantize_dual": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p, _c.c_void_p,
                                    _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_float, _c.c_void_p]),
    "mx_quantize_dual_sr": (_c.c_int, [_c.c_void_p, _c.c_int64, _c.c_int64, _c.c_int64, _c.c_void_p, _c.c_void_p,
                                       _c.c_void_p, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_float, _c.c_uint64,
                                       _c.c_uint64, _c.c_void_p]),
    "mx_gemm": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64,
                           _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p]),
    "mx_gemm_gelu_quantize": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64,
                                         _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_void_p, _c.c_void_p,
                                         _c.c_void_p]),
    "mx_gemm_ws": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64,
                              _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p, _c.c_size_t,
                              _c.c_void_p]),
    "mx_gemm_workspace_bytes": (_c.c_size_t, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "mx_gemm_scratch": (_c.c_int, [_c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_void_p, _c.c_int64,
                                   _c.c_int64, _c.c_int64, _c.c_int, _c.c_void_p, _c.c_int, _c.c_void_p]),
    "mx_gemm_plan": (_c.c_char_p, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int]),
    "mx_gemm_ws_plan": (_c.c_char_p, [_c.c_int64, _c.c_int64, _c.c_int64, _c.c_int, _c.c_size_t]),
    "mx_last_error": (_c.c_char_p, []),
}

_lib = None


def lib() -> ctypes.CDLL:
    """The loaded library; raises if it has not been built."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(
                f"{LIB_PATH} is missing: the HIP library must be built first "
                "(python -m block_scaled_precision_mx_amd.build)")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib
