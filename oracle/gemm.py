"""Dequantize-then-GEMM reference and the acceptance rule (test infrastructure only).

The product path computes C = A * B^T with both operands K-major ("TN"; the
lightly-train README "DINOv3 + EoMT on RTX 5090", section 5.5, writes every
low-precision GEMM this way), from operands quantized by the same format,
accumulating in fp32, then adds a bf16 bias and stores bf16 or fp32
(section 4.3 lists qkv / proj / fc1 / fc2 as the quantized GEMMs; section 4.3
and 5.7 describe the bias epilogues fused into them).

The oracle dequantizes both operands exactly into float64 and multiplies
with a plain float64 matmul; its own rounding error is at most about
K * 2^-53 * S, far below the acceptance bound 2^-12 * S, where
S[m, n] = sum_k |A[m, k] * B[n, k]| + |bias[n]|.

Acceptance (a reading: a bound stated on the exact sum cannot survive the
final bf16 rounding, which alone is 2^-9 relative, so the bound is applied
before that single rounding):
  * fp32 output:  |gpu - C_ref| <= 2^-12 * S
  * bf16 output:  RNE_bf16(C_ref - 2^-12 S) <= gpu <= RNE_bf16(C_ref + 2^-12 S)
    (RNE is monotone, so this says "gpu is the bf16 rounding of some value
    within the bound of the exact result").
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .quantize import Quantized

TOL = 2.0 ** -12


def gemm_ref(a: Quantized, b: Quantized, bias_bits=None):
    """C_ref [M, N] and S [M, N] in float64 for quantized A [M, K], B [N, K]."""
    if a.fmt != b.fmt:
        raise ValueError("operands must share a format")
    if a.length != b.length:
        raise ValueError("operands must share K")
    ah = a.dequantize()
    bh = b.dequantize()
    c = ah @ bh.T
    s = np.abs(ah) @ np.abs(bh).T
    if bias_bits is not None:
        bias = F.bf16_to_f64(np.asarray(bias_bits, dtype=np.uint16))
        c = c + bias[None, :]
        s = s + np.abs(bias)[None, :]
    return c, s


def gemm_ref_entries(a: Quantized, b: Quantized, rows, cols, bias_bits=None):
    """C_ref and S at sampled (row, col) pairs only, one dot product each."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    ah = a.dequantize()[rows]
    bh = b.dequantize()[cols]
    c = np.einsum("ik,ik->i", ah, bh)
    s = np.einsum("ik,ik->i", np.abs(ah), np.abs(bh))
    if bias_bits is not None:
        bias = F.bf16_to_f64(np.asarray(bias_bits, dtype=np.uint16))[cols]
        c = c + bias
        s = s + np.abs(bias)
    return c, s


def accept_bounds(c_ref, s, out_dtype: str):
    """(lo, hi) float64 bounds that a GPU output must lie within."""
    lo = c_ref - TOL * s
    hi = c_ref + TOL * s
    if out_dtype == "bf16":
        return F.f64_to_bf16_rne(lo), F.f64_to_bf16_rne(hi)
    if out_dtype == "f32":
        return lo, hi
    raise ValueError(f"unknown output dtype {out_dtype!r}")


def accept(gpu, c_ref, s, out_dtype: str) -> np.ndarray:
    """Boolean mask: which GPU outputs satisfy the acceptance rule."""
    lo, hi = accept_bounds(c_ref, s, out_dtype)
    g = np.asarray(gpu, dtype=np.float64)
    return (g >= lo) & (g <= hi)
