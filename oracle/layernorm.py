"""LayerNorm whose output leaves its kernel already quantized as the next
GEMM's operand (test infrastructure only: nothing on the product path
imports this module).

README "DINOv3 + EoMT on RTX 5090", section 4.3: in the MXFP8 stack
LayerNorm and quantization are one kernel (the block table's MXFP8 row;
section 4.6 lists the same fusion as planned work for the other stacks),
and the residual stream and the LayerNorm statistics stay fp32 in every
stack (section 4.1 and the text under its table).

Reading (the page names the fusion, not its arithmetic). The input is the
fp32 residual stream x [R, C]; gamma and beta are fp32 [C]; eps > 0. With
mu and var the mean and the biased variance of a row (nn.LayerNorm's
definition),

    y_i = (x_i - mu) / sqrt(var + eps) * gamma_i + beta_i,
    g   = RNE_bf16(y)             (the LayerNorm output as a bf16 tensor),

and the fused output is, byte for byte, what quantize(g, fmt, "row") gives:
the same bytes an LN kernel with bf16 output followed by mx_quantize would
write. y is computed in fp32 by the kernel, so it is not bit-fixed; it lies
within LN_REL * B_i of the exact value, where

    B_i = |gamma_i| r (max_j |x_j - mu| + |x_i - mu| + |mu|) + |beta_i| + |y_i|,
    r = 1 / sqrt(var + eps),

covering the fp32 rounding of the row sums (the mean's error scales with
the row's magnitude, the centred value's with |x_i - mu|), of the reciprocal
square root and of the final multiply-adds. A row sum of C fp32 terms taken
as C / 64 sequential terms per lane and then a 64-lane tree carries at most
about (C / 64 + 6) 2^-24 of the sum of magnitudes: a factor of about 4 to
spare at 4096 columns and about 2 at 8192, the widest row the kernel takes. Each element then has an interval of
possible bf16 values, and check_rows accepts an output iff some choice
inside the intervals explains every scale byte and code (fused.check_intervals).
"""
from __future__ import annotations

import numpy as np

from . import formats as F
from . import fused as FU
from . import quantize as Q

# allowance of the kernel's fp32 LayerNorm relative to B_i (see above)
LN_REL = 2.0 ** -16


def _stats(x: np.ndarray, eps: float):
    """Row mean, biased variance and 1 / sqrt(var + eps) in float64 (two
    passes; the fp32 inputs are exact in float64)."""
    x = np.asarray(x, dtype=np.float64)
    mu = x.mean(axis=1, keepdims=True)
    var = ((x - mu) ** 2).mean(axis=1, keepdims=True)
    return x, mu, var, 1.0 / np.sqrt(var + eps)


def layernorm(x, gamma, beta, eps: float) -> np.ndarray:
    """Exact (float64) LayerNorm of the rows of fp32 x [R, C]."""
    x, mu, _, r = _stats(x, eps)
    return (x - mu) * r * np.asarray(gamma, np.float64) + np.asarray(beta, np.float64)


def tolerance(x, gamma, beta, eps: float) -> tuple[np.ndarray, np.ndarray]:
    """(y exact, LN_REL * B) per element, B as in the module docstring."""
    x, mu, _, r = _stats(x, eps)
    gamma = np.asarray(gamma, np.float64)
    beta = np.asarray(beta, np.float64)
    y = (x - mu) * r * gamma + beta
    d = np.abs(x - mu)
    bound = np.abs(gamma) * r * (d.max(axis=1, keepdims=True) + d + np.abs(mu)) + np.abs(beta) + np.abs(y)
    return y, LN_REL * bound


def reference_codes(x, gamma, beta, eps: float, fmt: str) -> Q.Quantized:
    """The fused output for the exact LayerNorm: quantize(RNE_bf16(y))."""
    return Q.quantize(F.f64_to_bf16_bits(layernorm(x, gamma, beta, eps)), fmt, "row")


def check_rows(codes_rows: np.ndarray, scales_rows: np.ndarray, x, gamma, beta, eps: float, fmt: str):
    """Accept / reject the fused output of the rows x [R, C] (unpacked
    codes [R, K_pad], scale bytes [R, K_pad / 32]); returns (ok_codes,
    ok_scales) boolean masks."""
    y, tol = tolerance(x, gamma, beta, eps)
    g_lo = F.f64_to_bf16_rne(y - tol)
    g_hi = F.f64_to_bf16_rne(y + tol)
    return FU.check_intervals(codes_rows, scales_rows, g_lo, g_hi, fmt, y.shape[1])
