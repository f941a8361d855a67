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
kernel's GELU within GELU_REL * |GELU| + GELU_ABS of the exact value,
with the sign of h (GELU(h) = h Phi(h) and Phi > 0). So every element has
an interval of possible bf16 g values, and check_intervals accepts a block
of the output iff ONE choice of values inside those intervals explains all
of it at once:
  * for the GPU's scale byte (shared exponent e), each element's possible
    values are cut down to those whose RNE code at e is the GPU's code, the
    sign of a zero code included (a negative value, or -0, gives the
    negative-zero code);
  * some choice among what is left has a block amax whose shared exponent
    is e, i.e. amax in [2^(e + emax), 2^(e + emax + 1)) (any amax below the
    upper end for e = -127).
The values are bf16 numbers, so each element's remaining set is an
interval of bf16 magnitudes [m_i, M_i], and the achievable block amax runs
from max_i m_i to max_i M_i: the block is explained iff max_i M_i reaches
the exponent's lower end and max_i m_i stays below its upper end.
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


# What the kernel's fp32 GELU may differ from the exact one by, as the C
# header states it: its fitted tail Q(z) = exp(-z^2/2) R(z) is within 2^-20
# relative in fp32 and the rounding of the exp2 argument adds up to about
# 2^-16 near z = 13 (GELU_REL); the exp2 factor may flush results below
# 2^-126 to zero, which happens only where exp(-z^2/2) < 2^-126, and there
# |GELU(h)| = z Q(z) < phi(z) = exp(-z^2/2) / sqrt(2 pi) < 2^-127 (the
# Mills-ratio bound Q(z) < phi(z) / z), so an absolute 2^-126 covers the
# flush (GELU_ABS). The result keeps the sign of h.
GELU_REL = 2.0 ** -14
GELU_ABS = 2.0 ** -126


def _bf16_interval_of_gelu(h_lo, h_hi):
    """bf16 interval [g_lo, g_hi] of RNE_bf16(fp32 GELU) for h in [h_lo, h_hi]
    (float64 bf16 values with signed zeros): GELU's image of the interval,
    widened by the allowance, and clipped at zero on the side that h's sign
    excludes (GELU(h) has the sign of h, -0 for h = -0)."""
    a, b = gelu(h_lo), gelu(h_hi)
    g_min = np.minimum(a, b)
    g_max = np.maximum(a, b)
    inside = (h_lo < GELU_ARGMIN) & (h_hi > GELU_ARGMIN)
    g_min = np.where(inside, gelu(GELU_ARGMIN) * (1 + 1e-12), g_min)
    lo = F.f64_to_bf16_rne(g_min - (GELU_REL * np.abs(g_min) + GELU_ABS))
    hi = F.f64_to_bf16_rne(g_max + (GELU_REL * np.abs(g_max) + GELU_ABS))
    # every h has sign bit 0: no negative g (lo at least +0)
    pos_only = ~np.signbit(h_lo)
    lo = np.where(pos_only & (np.signbit(lo) | (lo == 0)), 0.0, lo)
    # every h has sign bit 1: no positive g (hi at most -0)
    neg_only = np.signbit(h_hi)
    hi = np.where(neg_only & ~np.signbit(hi), -0.0, hi)
    return lo, hi


def reference_codes(h_bits: np.ndarray, fmt: str) -> Q.Quantized:
    """The fused output for given bf16 pre-activations h (exact GELU rounded
    once to bf16, then quantize along the rows)."""
    g = F.f64_to_bf16_bits(gelu(F.bf16_to_f64(h_bits)))
    return Q.quantize(g, fmt, "row")


def check_rows(codes_rows: np.ndarray, scales_rows: np.ndarray, c: np.ndarray, s: np.ndarray, fmt: str,
               n: int, gemm_tol: float = G.TOL, extra=0.0):
    """Accept / reject the fused output of some rows.

    codes_rows: [R, K_pad] element codes (unpacked, one per element) of the
    GPU output rows; scales_rows: [R, K_pad / 32] scale bytes; c, s: [R, n]
    exact (acc + bias) and S of those rows; `extra` [R, n] (or a scalar) widens
    the GEMM allowance (the MXFP8 matrix instruction's adder term H of
    oracle.gemm). Returns (ok_codes [R, K_pad], ok_scales [R, K_pad / 32])
    boolean masks."""
    if fmt not in ("mxfp8", "mxfp4"):
        raise ValueError("the fused path emits MX formats")
    h_lo = F.f64_to_bf16_rne(c - gemm_tol * s - extra)
    h_hi = F.f64_to_bf16_rne(c + gemm_tol * s + extra)
    g_lo, g_hi = _bf16_interval_of_gelu(h_lo, h_hi)
    return check_intervals(codes_rows, scales_rows, g_lo, g_hi, fmt, n)


def _preimage(fmt):
    """Per magnitude code k: (low end, high end, ends inclusive) of the scaled
    magnitudes |x| 2^-e that round to k: the midpoints to the neighbours,
    inclusive for an even code (ties go to it), exclusive for an odd one; 0
    below code 0 and +inf above the largest code (saturation)."""
    grid = F.E4M3_GRID if fmt == "mxfp8" else F.E2M1_GRID
    mids = (grid[:-1] + grid[1:]) * 0.5
    low = np.concatenate([[0.0], mids])
    high = np.concatenate([mids, [np.inf]])
    even = (np.arange(grid.size) % 2) == 0
    return low, high, even


def check_intervals(codes_rows: np.ndarray, scales_rows: np.ndarray, g_lo: np.ndarray, g_hi: np.ndarray, fmt: str,
                    n: int):
    """Accept / reject MX row-quantized rows whose bf16 source values are
    known only to lie in [g_lo, g_hi] (float64 [R, n], bf16 values; a
    negative value is possible iff g_lo has its sign bit set, a positive one
    iff g_hi has not), the columns n .. K_pad being padding (+0, code 0).

    Returns (ok_codes [R, K_pad], ok_scales [R, K_pad / 32]): ok_codes says
    that some value of the element's interval has the GPU's code at the GPU's
    block exponent; ok_scales that one choice of such values gives the block
    an amax whose shared exponent is the GPU's (module docstring)."""
    if fmt not in ("mxfp8", "mxfp4"):
        raise ValueError("interval acceptance is defined for the MX formats")
    emax = F.E4M3_EMAX if fmt == "mxfp8" else F.E2M1_EMAX
    sign_shift, mag_mask = (7, 0x7F) if fmt == "mxfp8" else (3, 0x7)
    R, k_pad = codes_rows.shape
    nb = k_pad // 32
    lo = np.zeros((R, k_pad))
    hi = np.zeros((R, k_pad))
    lo[:, :n], hi[:, :n] = g_lo, g_hi
    codes = np.asarray(codes_rows, dtype=np.int64)
    e = scales_rows.astype(np.int64) - 127                      # [R, nb]
    e_el = np.repeat(e, 32, axis=1)
    neg = ((codes >> sign_shift) & 1) == 1
    k = codes & mag_mask
    top = (F.E4M3_GRID.size if fmt == "mxfp8" else F.E2M1_GRID.size) - 1
    valid = k <= top                                             # 0x7F is NaN in E4M3
    k = np.minimum(k, top)
    # magnitudes the interval allows with the code's sign
    sign_ok = np.where(neg, np.signbit(lo), ~np.signbit(hi))
    cm_lo = np.where(neg, np.where(hi < 0, -hi, 0.0), np.where(lo > 0, lo, 0.0))
    cm_hi = np.where(neg, -lo, hi)
    # magnitudes that round to k at exponent e, as bf16 values
    p_low, p_high, p_even = _preimage(fmt)
    low, high, incl = np.ldexp(p_low[k], e_el), np.ldexp(p_high[k], e_el), p_even[k]
    a = np.maximum(cm_lo, np.where(incl, F.bf16_ceil(low), F.bf16_above(low)))
    b = np.minimum(cm_hi, np.where(incl, F.bf16_floor(high), F.bf16_below(high)))
    ok_codes = valid & sign_ok & (a <= b)
    # the block amax that such a choice can reach: [max m_i, max M_i]
    m_blk = np.where(ok_codes, a, 0.0).reshape(R, nb, 32).max(axis=2)
    M_blk = np.where(ok_codes, b, 0.0).reshape(R, nb, 32).max(axis=2)
    amax_lo = np.where(e > -127, np.ldexp(1.0, e + emax), 0.0)   # e = -127 takes every amax below 2^(emax - 126)
    amax_hi = np.where(e < 127, np.ldexp(1.0, e + emax + 1), np.inf)
    ok_scales = (e >= -127) & (e <= 127) & (M_blk >= amax_lo) & (m_blk < amax_hi)
    ok_codes[:, n:] &= (codes_rows[:, n:] == 0)          # padding codes are +0
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
