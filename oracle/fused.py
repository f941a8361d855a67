"""fc1 -> GELU -> fc2's operand: a GEMM whose output leaves the producer
already quantized (test infrastructure only).

README "DINOv3 + EoMT on RTX 5090", section 4.3 (the block table, MXFP8
row): fc1's epilogue quantizes the GELU output straight into fc2's E4M3
operand, so the MXFP8 layer needs no separate quantization of the MLP
activation; section 4.6 lists the same fusion as planned work for the other
stacks.

Reading (the page names the fusion, not its arithmetic). The fused output is,
byte for byte, the row quantization (along N) that quantize() gives for

    g = RNE_bf16(GELU(h)),  h = RNE_bf16(acc + bias[n]),

where acc is the GEMM's fp32 accumulation (mx_gemm's, within 2^-12 S of the
exact sum, S = sum |a b| + |bias|) and GELU is the exact one,
GELU(h) = h Phi(h) = h/2 erfc(-h / sqrt 2). So the fused result equals
mx_quantize of the bf16 GELU of mx_gemm's bf16 output. Neither acc nor the
kernel's fp32 GELU is bit-fixed: acc lies within the GEMM bound, and the
kernel's GELU within GELU_REL * |GELU| + GELU_ABS of the exact value. So
every element has an interval of possible bf16 g values, and check() accepts
an output iff some choice inside those intervals explains it:
  * the block's scale byte lies between the shared exponents of the smallest
    and the largest possible block amax;
  * every code equals, at that scale, the RNE code of some value of its
    element's interval (RNE onto the grid is monotone, so the interval's end
    codes bound it).
With an exactly representable accumulation (gemm_tol 0) the intervals come
from the GELU allowance alone and almost every element has one candidate.
"""
from __future__ import annotations

import numpy as np
from scipy.optimize import brentq
from scipy.special import erfc

from . import formats as F
from . import gemm as G
from . import quantize as Q

SQRT1_2 = np.sqrt(0.5)


def _gelu_slope(x: float) -> float:
    """d/dx GELU = Phi(x) + x phi(x)."""
    return 0.5 * erfc(-x * SQRT1_2) + x * np.exp(-0.5 * x * x) / np.sqrt(2 * np.pi)


# GELU's single minimum: the root of its slope in [-1, -0.5]
GELU_ARGMIN = brentq(_gelu_slope, -1.0, -0.5, xtol=1e-15)


def gelu(h) -> np.ndarray:
    """Exact GELU in float64: h * Phi(h) = h / 2 * erfc(-h / sqrt 2)."""
    h = np.asarray(h, dtype=np.float64)
    return 0.5 * h * erfc(-h * SQRT1_2)


# what the kernel's fp32 GELU may differ from the exact one by: its fitted
# tail Q(z) = exp(-z^2/2) R(z) is within 2^-20 relative in fp32, the
# rounding of the exp2 argument adds up to about 2^-16 near z = 13, and the
# exp2 of arguments below -126 (|GELU| < 2^-122) may flush to zero
GELU_REL = 2.0 ** -14
GELU_ABS = 2.0 ** -122


def _bf16_interval_of_gelu(h_lo, h_hi):
    """bf16 interval [g_lo, g_hi] of RNE_bf16(fp32 GELU) for h in [h_lo, h_hi]."""
    a, b = gelu(h_lo), gelu(h_hi)
    g_min = np.minimum(a, b)
    g_max = np.maximum(a, b)
    inside = (h_lo < GELU_ARGMIN) & (h_hi > GELU_ARGMIN)
    g_min = np.where(inside, gelu(GELU_ARGMIN) * (1 + 1e-12), g_min)
    lo = g_min - (GELU_REL * np.abs(g_min) + GELU_ABS)
    hi = g_max + (GELU_REL * np.abs(g_max) + GELU_ABS)
    return F.f64_to_bf16_rne(lo), F.f64_to_bf16_rne(hi)


def reference_codes(h_bits: np.ndarray, fmt: str) -> Q.Quantized:
    """The fused output for given bf16 pre-activations h (exact GELU rounded
    once to bf16, then quantize along the rows)."""
    g = F.f64_to_bf16_bits(gelu(F.bf16_to_f64(h_bits)))
    return Q.quantize(g, fmt, "row")


def _enc_value(v, e, fmt):
    """Value of the RNE code of v at shared exponent e (saturating)."""
    scaled = np.ldexp(v, -e)
    if fmt == "mxfp8":
        return np.ldexp(F.e4m3_decode(F.e4m3_encode(scaled)), e)
    return np.ldexp(F.e2m1_decode(F.e2m1_encode(scaled)), e)


def check_rows(codes_rows: np.ndarray, scales_rows: np.ndarray, c: np.ndarray, s: np.ndarray, fmt: str,
               n: int, gemm_tol: float = G.TOL):
    """Accept / reject the fused output of some rows.

    codes_rows: [R, K_pad] element codes (unpacked, one per element) of the
    GPU output rows; scales_rows: [R, K_pad / 32] scale bytes; c, s: [R, n]
    exact (acc + bias) and S of those rows. Returns (ok_codes [R, K_pad],
    ok_scales [R, K_pad / 32]) boolean masks."""
    if fmt not in ("mxfp8", "mxfp4"):
        raise ValueError("the fused path emits MX formats")
    h_lo = F.f64_to_bf16_rne(c - gemm_tol * s)
    h_hi = F.f64_to_bf16_rne(c + gemm_tol * s)
    g_lo, g_hi = _bf16_interval_of_gelu(h_lo, h_hi)
    return check_intervals(codes_rows, scales_rows, g_lo, g_hi, fmt, n)


def check_intervals(codes_rows: np.ndarray, scales_rows: np.ndarray, g_lo: np.ndarray, g_hi: np.ndarray, fmt: str,
                    n: int):
    """Accept / reject MX row-quantized rows whose bf16 source values are
    known only to lie in [g_lo, g_hi] (float64 [R, n], bf16 values), the
    columns n .. K_pad being padding. Returns (ok_codes [R, K_pad],
    ok_scales [R, K_pad / 32]) boolean masks."""
    if fmt not in ("mxfp8", "mxfp4"):
        raise ValueError("interval acceptance is defined for the MX formats")
    emax = F.E4M3_EMAX if fmt == "mxfp8" else F.E2M1_EMAX
    R, k_pad = codes_rows.shape
    nb = k_pad // 32
    lo = np.zeros((R, k_pad))
    hi = np.zeros((R, k_pad))
    lo[:, :n], hi[:, :n] = g_lo, g_hi
    g_lo, g_hi = lo, hi
    # block amax range
    amin = np.where((g_lo <= 0) & (g_hi >= 0), 0.0, np.minimum(np.abs(g_lo), np.abs(g_hi)))
    amax = np.maximum(np.abs(g_lo), np.abs(g_hi))
    e_lo = Q.mx_shared_exponent(amin.reshape(R, nb, 32).max(axis=2), emax)
    e_hi = Q.mx_shared_exponent(amax.reshape(R, nb, 32).max(axis=2), emax)
    e_gpu = scales_rows.astype(np.int64) - 127
    ok_scales = (e_gpu >= e_lo) & (e_gpu <= e_hi)
    e_el = np.repeat(e_gpu, 32, axis=1)
    got = (F.e4m3_decode(codes_rows) if fmt == "mxfp8" else F.e2m1_decode(codes_rows))
    got = np.ldexp(got, e_el)
    lo_v = _enc_value(g_lo, e_el, fmt)
    hi_v = _enc_value(g_hi, e_el, fmt)
    ok_codes = (got >= lo_v) & (got <= hi_v)
    ok_codes[:, n:] &= (codes_rows[:, n:] == 0)          # padding codes are zero
    return ok_codes, ok_scales


def unpack_codes(packed_rows: np.ndarray, fmt: str) -> np.ndarray:
    """One code per element from stored rows (fp4: low nibble first)."""
    packed_rows = np.asarray(packed_rows, dtype=np.uint8)
    if fmt == "mxfp8":
        return packed_rows
    out = np.empty((packed_rows.shape[0], packed_rows.shape[1] * 2), dtype=np.uint8)
    out[:, 0::2] = packed_rows & 0xF
    out[:, 1::2] = packed_rows >> 4
    return out
