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

MXFP8 adds one term to that bound, H (mxfp8_group_term). It is not part of
the method: MI355X's scaled matrix instruction with E4M3 operands adds the
products of each group of 8 consecutive K elements in a fixed-point adder
that keeps 13 bits below the binade of the group's largest product and
truncates every other product toward zero (measured on the GPU with crafted
operands; the GPU test test_gpu_mfma_adder.py pins it). A product of two
E4M3 values has 8 significant bits, so products within 2^5 of the group's
largest are exact; smaller ones lose up to 2^(E_g - 13) each, E_g the
exponent of the group's largest product. So the instruction can be off the
exact sum by up to H = sum_g 7 * 2^(E_g - 13) <= 7 * 2^-13 * S ~ 2^-10.2 S,
which exceeds 2^-12 S only where a group mixes magnitudes (an outlier next to
ordinary values). E2M1 products span at most 144x within a block, and NVFP4's
fp16 operands go through another instruction, so those formats carry no such
term.
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from .quantize import Quantized

TOL = 2.0 ** -12
# the MXFP8 matrix instruction's adder: groups of 8 K elements, 13 bits kept
# below the binade of each group's largest product
MXFP8_GROUP = 8
MXFP8_GROUP_BITS = 13


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


def mxfp8_group_term(a: Quantized, b: Quantized, rows, cols) -> np.ndarray:
    """H at the (rows[i], cols[i]) entries of an MXFP8 GEMM (0 for the other
    formats): sum over the groups of 8 consecutive K elements of
    7 * 2^(E_g - 13), E_g = floor(log2 max_g |a_k b_k|) (module docstring)."""
    rows = np.asarray(rows)
    cols = np.asarray(cols)
    if a.fmt != "mxfp8":
        return np.zeros(rows.shape)
    ah = a.dequantize()[rows]
    bh = b.dequantize()[cols]
    k = ah.shape[1]
    pad = (-k) % MXFP8_GROUP
    p = np.abs(np.pad(ah * bh, ((0, 0), (0, pad))))
    gmax = p.reshape(len(rows), -1, MXFP8_GROUP).max(axis=2)
    _, e = np.frexp(gmax)                      # gmax = f 2^e, f in [0.5, 1): floor(log2) = e - 1
    term = np.where(gmax > 0, (MXFP8_GROUP - 1) * np.ldexp(1.0, e - 1 - MXFP8_GROUP_BITS), 0.0)
    return term.sum(axis=1)


def accept_bounds(c_ref, s, out_dtype: str, extra=0.0):
    """(lo, hi) float64 bounds that a GPU output must lie within; `extra` is
    added to the 2^-12 S allowance (the MXFP8 term H)."""
    lo = c_ref - TOL * s - extra
    hi = c_ref + TOL * s + extra
    if out_dtype == "bf16":
        return F.f64_to_bf16_rne(lo), F.f64_to_bf16_rne(hi)
    if out_dtype == "f32":
        return lo, hi
    raise ValueError(f"unknown output dtype {out_dtype!r}")


def accept(gpu, c_ref, s, out_dtype: str, extra=0.0) -> np.ndarray:
    """Boolean mask: which GPU outputs satisfy the acceptance rule."""
    lo, hi = accept_bounds(c_ref, s, out_dtype, extra)
    g = np.asarray(gpu, dtype=np.float64)
    return (g >= lo) & (g <= hi)


def accept_entries(gpu, c_ref, s, out_dtype: str, a: Quantized, b: Quantized, rows, cols) -> np.ndarray:
    """accept() for the entries (rows[i], cols[i]) of a GEMM of a and b, with
    the MXFP8 term H added (computed only where 2^-12 S alone rejects)."""
    gpu, c_ref, s = (np.asarray(v, dtype=np.float64).reshape(-1) for v in (gpu, c_ref, s))
    ok = accept(gpu, c_ref, s, out_dtype)
    if a.fmt == "mxfp8" and not ok.all():
        idx = np.flatnonzero(~ok)
        h = mxfp8_group_term(a, b, np.asarray(rows).reshape(-1)[idx], np.asarray(cols).reshape(-1)[idx])
        ok[idx] = accept(gpu[idx], c_ref[idx], s[idx], out_dtype, h)
    return ok
