"""MI355X-native block-scaled (MXFP8 / MXFP4 / NVFP4) quantize-then-GEMM.

The compute lives in libmx.so (hand-written HIP for gfx950, C ABI declared in
include/mx.h); ``api`` binds it for PyTorch device tensors.
"""
from ._lib import LIB_PATH, lib  # noqa: F401


def __getattr__(name):
    if name in ("mx_quantize", "mx_gemm", "Quantized", "codes_bytes", "scales_bytes", "k_pad", "MxError", "gemm_plan"):
        from . import api
        return getattr(api, name)
    raise AttributeError(name)
