"""Python binding of libmx with the C ABI's names (marshalling only).

Tensors are PyTorch device tensors; every step of quantization and GEMM
runs in the HIP library. Calls are enqueued on the current torch stream.
"""
from __future__ import annotations

from dataclasses import dataclass

import torch

from ._lib import lib

FMT = {"mxfp8": 1, "mxfp4": 2, "nvfp4": 3}
AXIS = {"row": 0, "col": 1}
OUT = {"bf16": 0, "f32": 1}
STATUS = {0: "MX_OK", 1: "MX_ERR_INVALID_ARG", 2: "MX_ERR_UNSUPPORTED", 3: "MX_ERR_ALIGNMENT", 4: "MX_ERR_HIP"}


class MxError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS.get(status, status)}: {message}")
        self.status = status


def _check(status: int) -> None:
    if status != 0:
        raise MxError(status, lib().mx_last_error().decode())


def _ld(x: torch.Tensor) -> int:
    """Leading dimension in elements (a single row's stride is arbitrary)."""
    return x.stride(0) if x.shape[0] > 1 else x.shape[1]


def _stream(stream) -> int:
    s = torch.cuda.current_stream() if stream is None else stream
    return s.cuda_stream


@dataclass
class Quantized:
    """Codes and scales of one operand: `rows` stored rows of `length` elements."""
    codes: torch.Tensor
    scales: torch.Tensor
    fmt: str
    rows: int
    length: int


def k_pad(length: int) -> int:
    return lib().mx_k_pad(length)


def gemm_plan(M: int, N: int, K: int, fmt: str) -> str:
    """Kernel configuration mx_gemm launches for these sizes (for profiling)."""
    name = lib().mx_gemm_plan(M, N, K, FMT[fmt])
    if name is None:
        raise ValueError("invalid GEMM sizes or format")
    return name.decode()


def gemm_workspace_bytes(M: int, N: int, K: int, fmt: str) -> int:
    """Workspace bytes with which mx_gemm_ws runs its fastest plan (0: no split)."""
    return lib().mx_gemm_workspace_bytes(M, N, K, FMT[fmt])


def gemm_ws_plan(M: int, N: int, K: int, fmt: str, workspace_bytes: int) -> str:
    """Kernel configuration mx_gemm_ws launches with that much workspace."""
    name = lib().mx_gemm_ws_plan(M, N, K, FMT[fmt], workspace_bytes)
    if name is None:
        raise ValueError("invalid GEMM sizes or format")
    return name.decode()


def codes_bytes(rows: int, cols: int, fmt: str, axis: str = "row") -> int:
    return lib().mx_codes_bytes(rows, cols, FMT[fmt], AXIS[axis])


def scales_bytes(rows: int, cols: int, fmt: str, axis: str = "row") -> int:
    return lib().mx_scales_bytes(rows, cols, FMT[fmt], AXIS[axis])


def mx_quantize(x: torch.Tensor, fmt: str, axis: str = "row", codes: torch.Tensor | None = None,
                scales: torch.Tensor | None = None, stream=None) -> Quantized:
    """Quantize a 2-D bf16 device tensor (unit column stride) along `axis`."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D bfloat16 device tensor")
    if x.stride(1) != 1 and x.shape[1] > 1:
        raise ValueError("x must have unit stride along its last dimension")
    rows, cols = x.shape
    nc, ns = codes_bytes(rows, cols, fmt, axis), scales_bytes(rows, cols, fmt, axis)
    if codes is None:
        codes = torch.empty(nc, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(ns, dtype=torch.uint8, device=x.device)
    if codes.numel() < nc or scales.numel() < ns:
        raise ValueError("codes / scales buffers are too small")
    _check(lib().mx_quantize(x.data_ptr(), rows, cols, _ld(x), codes.data_ptr(), scales.data_ptr(),
                             FMT[fmt], AXIS[axis], _stream(stream)))
    stored_rows, length = (rows, cols) if axis == "row" else (cols, rows)
    return Quantized(codes, scales, fmt, stored_rows, length)


def mx_quantize_batch(xs: list[torch.Tensor], fmt: str, out: list[Quantized] | None = None,
                      stream=None, amax: torch.Tensor | None = None) -> list[Quantized]:
    """Row quantization of several 2-D bf16 device tensors in one launch
    (MXFP8 / MXFP4; at most QUANT_BATCH_MAX tensors per call). `out` reuses
    the buffers of an earlier call's result. With `amax` (a float32 device
    tensor of len(xs) * AMAX_WORDS elements) the call is
    mx_quantize_batch_amax: each tensor's amax is also reduced, tensor i into
    amax[i * AMAX_WORDS:(i + 1) * AMAX_WORDS], for mx_quantize_amax."""
    from ._lib import AMAX_WORDS, QUANT_BATCH_MAX, QuantItem
    if not 1 <= len(xs) <= QUANT_BATCH_MAX:
        raise ValueError(f"between 1 and {QUANT_BATCH_MAX} tensors per call")
    if amax is not None and (amax.dtype != torch.float32 or not amax.is_cuda or not amax.is_contiguous()
                             or amax.numel() < len(xs) * AMAX_WORDS):
        raise ValueError(f"amax must be a contiguous float32 device tensor of {len(xs) * AMAX_WORDS} elements")
    items = (QuantItem * len(xs))()
    result = []
    for i, x in enumerate(xs):
        if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
            raise ValueError("every tensor must be a 2-D bfloat16 device tensor")
        if x.stride(1) != 1 and x.shape[1] > 1:
            raise ValueError("every tensor must have unit stride along its last dimension")
        rows, cols = x.shape
        nc, ns = codes_bytes(rows, cols, fmt, "row"), scales_bytes(rows, cols, fmt, "row")
        if out is None:
            q = Quantized(torch.empty(nc, dtype=torch.uint8, device=x.device),
                          torch.empty(ns, dtype=torch.uint8, device=x.device), fmt, rows, cols)
        else:
            q = out[i]
            if q.codes.numel() < nc or q.scales.numel() < ns:
                raise ValueError("out buffers are too small")
        items[i] = QuantItem(x.data_ptr(), rows, cols, _ld(x), q.codes.data_ptr(), q.scales.data_ptr())
        result.append(Quantized(q.codes, q.scales, fmt, rows, cols))
    if amax is None:
        _check(lib().mx_quantize_batch(items, len(xs), FMT[fmt], _stream(stream)))
    else:
        _check(lib().mx_quantize_batch_amax(items, len(xs), FMT[fmt], amax.data_ptr(), _stream(stream)))
    return result


def mx_quantize_amax(x: torch.Tensor, fmt: str, axis: str, amax: torch.Tensor, codes: torch.Tensor | None = None,
                     scales: torch.Tensor | None = None, stream=None) -> Quantized:
    """mx_quantize (NVFP4) with the tensor amax given: the largest magnitude
    among the elements of `amax` (a contiguous float32 device tensor of 1 ..
    AMAX_MAX_WORDS elements, e.g. one tensor's slice of mx_quantize_batch's
    `amax`)."""
    from ._lib import AMAX_MAX_WORDS
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D bfloat16 device tensor")
    if x.stride(1) != 1 and x.shape[1] > 1:
        raise ValueError("x must have unit stride along its last dimension")
    if amax.dtype != torch.float32 or not amax.is_cuda or not amax.is_contiguous() or \
            not 1 <= amax.numel() <= AMAX_MAX_WORDS:
        raise ValueError(f"amax must be a contiguous float32 device tensor of 1 .. {AMAX_MAX_WORDS} elements")
    rows, cols = x.shape
    nc, ns = codes_bytes(rows, cols, fmt, axis), scales_bytes(rows, cols, fmt, axis)
    if codes is None:
        codes = torch.empty(nc, dtype=torch.uint8, device=x.device)
    if scales is None:
        scales = torch.empty(ns, dtype=torch.uint8, device=x.device)
    if codes.numel() < nc or scales.numel() < ns:
        raise ValueError("codes / scales buffers are too small")
    _check(lib().mx_quantize_amax(x.data_ptr(), rows, cols, _ld(x), codes.data_ptr(), scales.data_ptr(),
                                  FMT[fmt], AXIS[axis], amax.data_ptr(), amax.numel(), _stream(stream)))
    stored_rows, length = (rows, cols) if axis == "row" else (cols, rows)
    return Quantized(codes, scales, fmt, stored_rows, length)


def mx_layernorm_quantize(x: torch.Tensor, gamma: torch.Tensor, beta: torch.Tensor, eps: float, fmt: str,
                          out: Quantized | None = None, stream=None) -> Quantized:
    """LayerNorm of the rows of a 2-D fp32 device tensor (the residual
    stream; gamma, beta fp32 [cols]) rounded to bf16 and row-quantized in
    one launch (MXFP8 / MXFP4): the operand of the next GEMM."""
    if x.dtype != torch.float32 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D float32 device tensor")
    if x.stride(1) != 1 and x.shape[1] > 1:
        raise ValueError("x must have unit stride along its last dimension")
    rows, cols = x.shape
    for name, t in (("gamma", gamma), ("beta", beta)):
        if t.dtype != torch.float32 or t.numel() != cols or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous float32 device tensor of {cols} elements")
    nc, ns = codes_bytes(rows, cols, fmt, "row"), scales_bytes(rows, cols, fmt, "row")
    if out is None:
        out = Quantized(torch.empty(nc, dtype=torch.uint8, device=x.device),
                        torch.empty(ns, dtype=torch.uint8, device=x.device), fmt, rows, cols)
    elif out.codes.numel() < nc or out.scales.numel() < ns:
        raise ValueError("out buffers are too small")
    _check(lib().mx_layernorm_quantize(x.data_ptr(), rows, cols, _ld(x), gamma.data_ptr(), beta.data_ptr(),
                                       float(eps), out.codes.data_ptr(), out.scales.data_ptr(), FMT[fmt],
                                       _stream(stream)))
    return Quantized(out.codes, out.scales, fmt, rows, cols)


def mx_quantize_dual(x: torch.Tensor, fmt: str, amax_prev: torch.Tensor | None = None, headroom: float = 32.0,
                     out: tuple[Quantized, Quantized] | None = None, stream=None) -> tuple[Quantized, Quantized]:
    """Row copy and transposed (column) copy of a 2-D bf16 device tensor from
    one read. NVFP4: amax_prev (a device float32 tensor of one element, e.g.
    amax_field(previous.scales)) selects the delayed tensor scale. `out`
    reuses the buffers of an earlier call's result."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D bfloat16 device tensor")
    if x.stride(1) != 1 and x.shape[1] > 1:
        raise ValueError("x must have unit stride along its last dimension")
    ptr = 0
    if amax_prev is not None:
        if amax_prev.dtype != torch.float32 or amax_prev.numel() < 1 or not amax_prev.is_cuda:
            raise ValueError("amax_prev must be a float32 device tensor")
        ptr = amax_prev.data_ptr()
    rows, cols = x.shape
    bufs = []
    for i, axis in enumerate(("row", "col")):
        nc, ns = codes_bytes(rows, cols, fmt, axis), scales_bytes(rows, cols, fmt, axis)
        if out is None:
            bufs.append(torch.empty(nc, dtype=torch.uint8, device=x.device))
            bufs.append(torch.empty(ns, dtype=torch.uint8, device=x.device))
        else:
            if out[i].codes.numel() < nc or out[i].scales.numel() < ns:
                raise ValueError("out buffers are too small")
            bufs += [out[i].codes, out[i].scales]
    _check(lib().mx_quantize_dual(x.data_ptr(), rows, cols, _ld(x), bufs[0].data_ptr(), bufs[1].data_ptr(),
                                  bufs[2].data_ptr(), bufs[3].data_ptr(), FMT[fmt], ptr or None, float(headroom),
                                  _stream(stream)))
    return (Quantized(bufs[0], bufs[1], fmt, rows, cols), Quantized(bufs[2], bufs[3], fmt, cols, rows))


def mx_quantize_dual_sr(x: torch.Tensor, seed: tuple[int, int], amax_prev: torch.Tensor | None = None,
                        headroom: float = 32.0, out: tuple[Quantized, Quantized] | None = None,
                        stream=None) -> tuple[Quantized, Quantized]:
    """NVFP4 row and column copies of x with stochastically rounded elements
    (Philox4x64-10 draws keyed by seed = (k0, k1), one per element of x);
    scales, s_t and trailers as mx_quantize_dual. x.shape[1] % 8 == 0."""
    if x.dtype != torch.bfloat16 or x.dim() != 2 or not x.is_cuda:
        raise ValueError("x must be a 2-D bfloat16 device tensor")
    if x.stride(1) != 1 and x.shape[1] > 1:
        raise ValueError("x must have unit stride along its last dimension")
    ptr = 0
    if amax_prev is not None:
        if amax_prev.dtype != torch.float32 or amax_prev.numel() < 1 or not amax_prev.is_cuda:
            raise ValueError("amax_prev must be a float32 device tensor")
        ptr = amax_prev.data_ptr()
    fmt = "nvfp4"
    rows, cols = x.shape
    bufs = []
    for i, axis in enumerate(("row", "col")):
        nc, ns = codes_bytes(rows, cols, fmt, axis), scales_bytes(rows, cols, fmt, axis)
        if out is None:
            bufs.append(torch.empty(nc, dtype=torch.uint8, device=x.device))
            bufs.append(torch.empty(ns, dtype=torch.uint8, device=x.device))
        else:
            if out[i].codes.numel() < nc or out[i].scales.numel() < ns:
                raise ValueError("out buffers are too small")
            bufs += [out[i].codes, out[i].scales]
    k0, k1 = (int(v) & ((1 << 64) - 1) for v in seed)
    _check(lib().mx_quantize_dual_sr(x.data_ptr(), rows, cols, _ld(x), bufs[0].data_ptr(), bufs[1].data_ptr(),
                                     bufs[2].data_ptr(), bufs[3].data_ptr(), FMT[fmt], ptr or None, float(headroom),
                                     k0, k1, _stream(stream)))
    return (Quantized(bufs[0], bufs[1], fmt, rows, cols), Quantized(bufs[2], bufs[3], fmt, cols, rows))


def amax_field(scales: torch.Tensor) -> torch.Tensor:
    """The fp32 amax of an NVFP4 scale buffer's trailer, as a one-element view."""
    return scales[-16:].view(torch.float32)[1:2]


def mx_gemm(a: Quantized, b: Quantized, bias: torch.Tensor | None = None, out_dtype: str = "bf16",
            out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """C[M, N] = A * B^T (+ bias) from two operands quantized in one format."""
    if a.fmt != b.fmt or a.length != b.length:
        raise ValueError("operands must share format and K")
    M, N, K = a.rows, b.rows, a.length
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=a.codes.device)
    if out.dtype != dt or out.numel() < M * N or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of M*N elements of the output dtype")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bf16 tensor of N elements")
    _check(lib().mx_gemm(a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(), b.scales.data_ptr(),
                         out.data_ptr(), M, N, K, FMT[a.fmt], None if bias is None else bias.data_ptr(),
                         OUT[out_dtype], _stream(stream)))
    return out


def mx_gemm_ws(a: Quantized, b: Quantized, bias: torch.Tensor | None, out_dtype: str,
               workspace: torch.Tensor | None, out: torch.Tensor | None = None, stream=None) -> torch.Tensor:
    """mx_gemm that may split K over a device workspace (uint8 tensor, or None)."""
    if a.fmt != b.fmt or a.length != b.length:
        raise ValueError("operands must share format and K")
    M, N, K = a.rows, b.rows, a.length
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    if out is None:
        out = torch.empty((M, N), dtype=dt, device=a.codes.device)
    if out.dtype != dt or out.numel() < M * N or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of M*N elements of the output dtype")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bf16 tensor of N elements")
    ws_ptr, ws_bytes = (None, 0) if workspace is None else (workspace.data_ptr(), workspace.numel() * workspace.element_size())
    _check(lib().mx_gemm_ws(a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(), b.scales.data_ptr(),
                            out.data_ptr(), M, N, K, FMT[a.fmt], None if bias is None else bias.data_ptr(),
                            OUT[out_dtype], ws_ptr, ws_bytes, _stream(stream)))
    return out


def mx_gemm_scratch(a: Quantized, b: Quantized, bias: torch.Tensor | None, out_dtype: str,
                    out: torch.Tensor, stream=None) -> torch.Tensor:
    """mx_gemm_ws with the library's own device scratch (allocates nothing;
    `out` must be given)."""
    if a.fmt != b.fmt or a.length != b.length:
        raise ValueError("operands must share format and K")
    M, N, K = a.rows, b.rows, a.length
    dt = torch.bfloat16 if out_dtype == "bf16" else torch.float32
    if out.dtype != dt or out.numel() < M * N or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor of M*N elements of the output dtype")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bf16 tensor of N elements")
    _check(lib().mx_gemm_scratch(a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(), b.scales.data_ptr(),
                                 out.data_ptr(), M, N, K, FMT[a.fmt], None if bias is None else bias.data_ptr(),
                                 OUT[out_dtype], _stream(stream)))
    return out


def mx_gemm_gelu_quantize(a: Quantized, b: Quantized, bias: torch.Tensor | None = None,
                          out: Quantized | None = None, stream=None) -> Quantized:
    """GELU(A * B^T (+ bias)) row-quantized in the operands' MX format, ready
    to be the A operand of the next GEMM (K = N); the activation itself is
    never stored."""
    if a.fmt != b.fmt or a.length != b.length:
        raise ValueError("operands must share format and K")
    M, N, K = a.rows, b.rows, a.length
    nc, ns = codes_bytes(M, N, a.fmt, "row"), scales_bytes(M, N, a.fmt, "row")
    if out is None:
        out = Quantized(torch.empty(nc, dtype=torch.uint8, device=a.codes.device),
                        torch.empty(ns, dtype=torch.uint8, device=a.codes.device), a.fmt, M, N)
    elif out.codes.numel() < nc or out.scales.numel() < ns:
        raise ValueError("out buffers are too small")
    if bias is not None and (bias.dtype != torch.bfloat16 or bias.numel() != N or not bias.is_contiguous()):
        raise ValueError("bias must be a contiguous bf16 tensor of N elements")
    _check(lib().mx_gemm_gelu_quantize(a.codes.data_ptr(), a.scales.data_ptr(), b.codes.data_ptr(),
                                       b.scales.data_ptr(), M, N, K, FMT[a.fmt],
                                       None if bias is None else bias.data_ptr(), out.codes.data_ptr(),
                                       out.scales.data_ptr(), _stream(stream)))
    return Quantized(out.codes, out.scales, a.fmt, M, N)
