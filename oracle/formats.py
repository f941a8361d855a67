"""Number formats used by the oracle (test infrastructure only).

bf16: 1 sign, 8 exponent, 7 mantissa bits -- the bf16 row of the format table
in "2x, not 16x: the real ledger of BF16 mixed precision", section 2. A bf16
value is the upper half of an IEEE binary32, so decoding is exact in float64.

E4M3 (element of MXFP8, block scale of NVFP4): the OCP "E4M3FN" variant,
1 sign, 4 exponent (bias 7), 3 mantissa bits, subnormals m * 2^-9, no
infinities, NaN only at magnitude 0x7F. Its largest finite value is 448,
the figure stated in the same blog, section 5.4.

E2M1 (element of MXFP4 and NVFP4, lightly-train README section 2 table):
1 sign, 2 exponent (bias 1), 1 mantissa bit; magnitudes
{0, 0.5, 1, 1.5, 2, 3, 4, 6}; no infinities or NaN.

UE8M0 (MX block scale): unsigned exponent byte b meaning 2^(b-127).

Readings taken where the pages say nothing (each applied below):
  * rounding is round-to-nearest, ties to the even code (LSB 0);
  * magnitudes above the largest finite value saturate to it (no NaN/Inf);
  * the sign bit of the code is the sign bit of the input, so -0.0, or a
    negative value that rounds to zero, gives the negative-zero code.
"""
from __future__ import annotations

import math

import numpy as np

# ---------------------------------------------------------------- bf16


def bf16_to_f64(bits) -> np.ndarray:
    """Exact float64 values of bf16 bit patterns (uint16 array)."""
    bits = np.asarray(bits, dtype=np.uint16)
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def f64_to_bf16_rne(x) -> np.ndarray:
    """Round float64 values to the nearest bf16 value (ties to even), as float64.

    A single rounding straight from float64 (no float32 stop on the way, which
    could round twice). Magnitudes beyond the bf16 range become +-inf; values
    below the smallest bf16 subnormal spacing (2^-133) round on that grid.
    """
    x = np.asarray(x, dtype=np.float64)
    out = np.empty_like(x)
    mant, expo = np.frexp(x)  # x = mant * 2^expo, 0.5 <= |mant| < 1
    # bf16 keeps 8 significant bits: spacing is 2^(expo-8), but never finer
    # than the subnormal spacing 2^-133.
    spacing_exp = np.maximum(expo - 8, -133)
    q = np.ldexp(x, -spacing_exp)          # exact: power-of-two scaling
    r = np.rint(q)                         # numpy rint is round-half-even
    out[...] = np.ldexp(r, spacing_exp)
    out[x == 0] = x[x == 0]                # keep the sign of zero
    big = np.abs(out) > 3.3895313892515355e38   # above bf16 max (0x7F7F)
    out[big] = np.copysign(np.inf, x[big])
    return out


def _bf16_spacing_exp(x: np.ndarray) -> np.ndarray:
    """Exponent of the bf16 spacing at the magnitude of x (8 significant
    bits, never finer than the subnormal spacing 2^-133)."""
    _, expo = np.frexp(np.abs(x))
    return np.maximum(expo - 8, -133)


def bf16_floor(x) -> np.ndarray:
    """Largest bf16 value <= x, for finite x >= 0 (as float64; +inf stays)."""
    x = np.asarray(x, dtype=np.float64)
    q = _bf16_spacing_exp(np.where(np.isfinite(x), x, 0.0))
    out = np.ldexp(np.floor(np.ldexp(x, -q)), q)
    return np.where(np.isfinite(x), out, x)


def bf16_ceil(x) -> np.ndarray:
    """Smallest bf16 value >= x, for finite x >= 0 (as float64; +inf stays)."""
    x = np.asarray(x, dtype=np.float64)
    q = _bf16_spacing_exp(np.where(np.isfinite(x), x, 0.0))
    out = np.ldexp(np.ceil(np.ldexp(x, -q)), q)
    return np.where(np.isfinite(x), out, x)


def bf16_above(x) -> np.ndarray:
    """Smallest bf16 value > x, for finite x >= 0 (+inf stays). Scaling by
    1 + 2^-20 moves a bf16 value past itself but not past the next one."""
    x = np.asarray(x, dtype=np.float64)
    c = bf16_ceil(x)
    nxt = np.where(c > 0, bf16_ceil(c * (1 + 2.0 ** -20)), 2.0 ** -133)
    return np.where(c > x, c, nxt)


def bf16_below(x) -> np.ndarray:
    """Largest bf16 value < x, for x >= 0 (+inf stays; -1 where none, i.e.
    x = 0)."""
    x = np.asarray(x, dtype=np.float64)
    f = bf16_floor(x)
    prv = np.where(f > 0, bf16_floor(f * (1 - 2.0 ** -20)), -1.0)
    return np.where(f < x, f, prv)


def f64_to_bf16_bits(x) -> np.ndarray:
    """bf16 bit patterns of float64 values after a single RNE rounding."""
    r = f64_to_bf16_rne(x).astype(np.float32)   # exact: r already has 8 bits
    return (r.view(np.uint32) >> 16).astype(np.uint16)


# ---------------------------------------------------------------- grids


def _e4m3_magnitude(m: int) -> float:
    """Value of E4M3FN magnitude bits m (0..0x7E)."""
    exp_field, mant = m >> 3, m & 7
    if exp_field == 0:
        return mant * 2.0 ** -9
    return (1.0 + mant / 8.0) * 2.0 ** (exp_field - 7)


# Sorted non-negative finite grids; the index of a value is its magnitude code.
E4M3_GRID = np.array([_e4m3_magnitude(m) for m in range(0x7F)], dtype=np.float64)
E2M1_GRID = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], dtype=np.float64)

E4M3_MAX = 448.0
E2M1_MAX = 6.0
E4M3_EMAX = 8     # floor(log2(448))
E2M1_EMAX = 2     # floor(log2(6))


def e4m3_decode(codes) -> np.ndarray:
    """float64 values of E4M3FN codes (uint8). 0x7F/0xFF decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    val = np.where(mag == 0x7F, np.nan, E4M3_GRID[np.minimum(mag, 0x7E)])
    return np.where(c & 0x80, -val, val)


def e2m1_decode(codes) -> np.ndarray:
    """float64 values of E2M1 codes (uint8 holding 0..15)."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    val = E2M1_GRID[c & 7]
    return np.where(c & 8, -val, val)


def ue8m0_decode(b) -> np.ndarray:
    """float64 values 2^(b-127) of UE8M0 scale bytes."""
    return np.ldexp(1.0, np.asarray(b, dtype=np.int64) - 127)


# ---------------------------------------------------------------- encoders


def _rne_index(v: np.ndarray, grid: np.ndarray) -> np.ndarray:
    """Index of the RNE rounding of non-negative float64 v onto `grid`.

    grid is sorted, grid[0] == 0; values above grid[-1] saturate to the last
    index. Between neighbours g[i] < v < g[i+1] the nearer one wins; exactly
    at the midpoint the even index (code LSB 0) wins. The midpoint of two
    grid values with few significant bits is exact in float64.
    """
    v = np.asarray(v, dtype=np.float64)
    top = len(grid) - 1
    hi = np.searchsorted(grid, v, side="left")        # grid[hi-1] < v <= grid[hi]
    hi = np.clip(hi, 1, top)
    lo = hi - 1
    mid = (grid[lo] + grid[hi]) * 0.5
    pick_hi = (v > mid) | ((v == mid) & (hi % 2 == 0))
    idx = np.where(pick_hi, hi, lo)
    idx = np.where(v >= grid[top], top, idx)           # saturate
    idx = np.where(v <= 0.0, 0, idx)
    return idx.astype(np.int64)


def e4m3_encode(x) -> np.ndarray:
    """E4M3FN codes (uint8) of float64 x: RNE, saturate at +-448, sign copied."""
    x = np.asarray(x, dtype=np.float64)
    mag = _rne_index(np.abs(x), E4M3_GRID)
    sign = np.signbit(x).astype(np.int64) << 7
    return (sign | mag).astype(np.uint8)


def e2m1_encode(x) -> np.ndarray:
    """E2M1 codes (uint8, 0..15) of float64 x: RNE, saturate at +-6, sign copied."""
    x = np.asarray(x, dtype=np.float64)
    mag = _rne_index(np.abs(x), E2M1_GRID)
    sign = np.signbit(x).astype(np.int64) << 3
    return (sign | mag).astype(np.uint8)


def floor_log2(a: float) -> int:
    """Exact floor(log2(a)) of a positive finite float via its binary exponent."""
    m, e = math.frexp(a)     # a = m * 2^e, 0.5 <= m < 1
    return e - 1
