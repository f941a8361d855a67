"""Block-scaled quantization, the plain way (test infrastructure only).

What it computes (lightly-train README "DINOv3 + EoMT on RTX 5090"):
  * section 2 table: MXFP8 = E4M3 elements + UE8M0 scale per 1x32 block;
    MXFP4 = E2M1 + UE8M0 per 1x32; NVFP4 = E2M1 + E4M3 scale per 1x16 plus
    an fp32 per-tensor scale.
  * section 5.5: GEMMs are TN with K-major operands, and the weight-gradient
    GEMM takes a copy quantized along the token axis and stored transposed.
    Here axis="row" quantizes blocks along the contiguous (last) dimension of
    X [R, C]; axis="col" quantizes blocks along the first dimension, i.e. it
    is the row quantization of X transposed, and stores X^T's codes.

Readings where the pages are silent (listed with the others in the design
notes of the repository):
  * MX shared exponent e = floor(log2(block amax)) - emax_elem, emax 8 for
    E4M3 and 2 for E2M1, clamped to [-127, 127]; an all-zero block gets
    e = -127. The scale byte is e + 127.
  * MX elements are x * 2^-e rounded RNE onto the element grid, saturated.
  * NVFP4: s_t = fp32 round-to-nearest-even of tensor_amax / (448 * 6);
    block byte = E4M3 RNE of the exact real block_amax / (6 * s_t);
    element code = E2M1 RNE of the exact real x / (dec(byte) * s_t).
    If s_t or the block scale is zero, the codes are signed zeros.
  * the last block of a row may be partial (e.g. 11235 = 351*32 + 3); its
    amax is over the real elements only.
  * storage: the quantized length L is padded to K_pad = round_up(L, 128)
    with zero codes and zero scale bytes; fp4 element 2i sits in the low
    nibble of byte i, element 2i+1 in the high nibble; scales are a plain
    row-major [rows, K_pad / bs] byte array. For NVFP4 the scale buffer
    carries a 16-byte trailer {float32 s_t, float32 amax, 0, 0} placed at
    the first 16-byte boundary after the scale bytes.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np

from . import formats as F

FORMATS = ("mxfp8", "mxfp4", "nvfp4")
AXES = ("row", "col")
K_ALIGN = 128


def block_size(fmt: str) -> int:
    return 16 if fmt == "nvfp4" else 32


def round_up(n: int, m: int) -> int:
    return -(-n // m) * m


@dataclass
class Quantized:
    fmt: str
    rows: int          # rows of the stored (possibly transposed) operand
    length: int        # real number of elements along the block axis
    k_pad: int         # padded length
    codes: np.ndarray  # uint8, element codes unpacked: [rows, k_pad]
    scales: np.ndarray  # uint8 [rows, k_pad // bs]
    s_t: np.float32 = np.float32(0)    # NVFP4 only
    amax: np.float32 = np.float32(0)   # NVFP4 only

    def packed_codes(self) -> np.ndarray:
        """Codes as stored: 1 byte per fp8 element, 2 fp4 elements per byte."""
        if self.fmt == "mxfp8":
            return self.codes.copy()
        lo = self.codes[:, 0::2].astype(np.uint8)
        hi = self.codes[:, 1::2].astype(np.uint8)
        return (lo | (hi << 4)).astype(np.uint8)

    def scale_buffer(self) -> np.ndarray:
        """The scale buffer byte image, including the NVFP4 trailer."""
        flat = self.scales.reshape(-1)
        if self.fmt != "nvfp4":
            return flat.copy()
        n = round_up(flat.size, 16)
        out = np.zeros(n + 16, dtype=np.uint8)
        out[: flat.size] = flat
        out[n: n + 8] = np.array([self.s_t, self.amax], dtype=np.float32).view(np.uint8)
        return out

    def dequantize(self) -> np.ndarray:
        """Exact float64 values [rows, length] that the codes and scales stand for."""
        bs = block_size(self.fmt)
        if self.fmt == "mxfp8":
            elem = F.e4m3_decode(self.codes)
        else:
            elem = F.e2m1_decode(self.codes)
        if self.fmt == "nvfp4":
            blk = F.e4m3_decode(self.scales) * np.float64(self.s_t)
        else:
            blk = F.ue8m0_decode(self.scales)
        val = elem * np.repeat(blk, bs, axis=1)
        return val[:, : self.length]


def _view(bits: np.ndarray, axis: str) -> np.ndarray:
    bits = np.asarray(bits, dtype=np.uint16)
    if bits.ndim != 2:
        raise ValueError("expected a 2-D bf16 bit array")
    if axis == "row":
        return bits
    if axis == "col":
        return np.ascontiguousarray(bits.T)
    raise ValueError(f"unknown axis {axis!r}")


def _blocks(x: np.ndarray, bs: int, k_pad: int) -> np.ndarray:
    """float64 [rows, L] -> [rows, k_pad // bs, bs], zero-padded."""
    rows, length = x.shape
    padded = np.zeros((rows, k_pad), dtype=np.float64)
    padded[:, :length] = x
    return padded.reshape(rows, k_pad // bs, bs)


def mx_shared_exponent(block_amax: np.ndarray, emax: int) -> np.ndarray:
    """e = clamp(floor(log2 amax) - emax, -127, 127); amax == 0 -> -127."""
    a = np.asarray(block_amax, dtype=np.float64)
    _, ex = np.frexp(a)                   # a = m * 2^ex, 0.5 <= m < 1
    e = (ex.astype(np.int64) - 1) - emax  # floor(log2 a) = ex - 1
    e = np.clip(e, -127, 127)
    return np.where(a == 0.0, -127, e)


def _quantize_mx(x: np.ndarray, fmt: str, k_pad: int):
    bs = 32
    emax = F.E4M3_EMAX if fmt == "mxfp8" else F.E2M1_EMAX
    blocks = _blocks(x, bs, k_pad)
    amax = np.abs(blocks).max(axis=2)
    e = mx_shared_exponent(amax, emax)
    scales = (e + 127).astype(np.uint8)
    v = np.ldexp(blocks, -e[:, :, None])  # exact: scaling by a power of two
    enc = F.e4m3_encode if fmt == "mxfp8" else F.e2m1_encode
    codes = enc(v).reshape(x.shape[0], k_pad)
    return codes, scales


# E2M1 midpoints between neighbouring grid values, in grid order.
_E2M1_MIDS = (F.E2M1_GRID[:-1] + F.E2M1_GRID[1:]) * 0.5


def nvfp4_tensor_scale(tensor_amax: float) -> np.float32:
    """s_t = fp32 RNE of amax / 2688 (2688 = 448 * 6).

    The float64 quotient cannot sit within 2^-53 of an fp32 rounding boundary
    (amax has 8 significant bits and 1/21 has a period-6 binary expansion),
    so rounding float64 -> float32 here rounds the exact quotient once.
    """
    return np.float32(np.float64(tensor_amax) / 2688.0)


def nvfp4_block_bytes(block_amax: np.ndarray, s_t: np.float32) -> np.ndarray:
    """E4M3 RNE (saturating) of the exact real block_amax / (6 * s_t).

    Dividing by a positive constant preserves order and midpoints, so the
    byte is the RNE index of block_amax on the E4M3 grid multiplied by
    6 * s_t. Every grid value and midpoint of that scaled grid is exact in
    float64 (at most 5 + 26 significant bits).
    """
    a = np.asarray(block_amax, dtype=np.float64)
    if s_t == 0:
        return np.zeros(a.shape, dtype=np.uint8)
    grid = F.E4M3_GRID * (6.0 * np.float64(s_t))
    return F._rne_index(a, grid).astype(np.uint8)


def nvfp4_element_codes(x: np.ndarray, S: np.ndarray) -> np.ndarray:
    """E2M1 RNE (saturating) of the exact real x / S, sign copied from x.

    Compares |x| with the seven E2M1 midpoints times S, each product exact in
    float64. Crossing midpoint i moves the code from i to i+1; a value equal
    to midpoint i goes to whichever of i, i+1 is even. S == 0 gives zeros.
    """
    x = np.asarray(x, dtype=np.float64)
    S = np.asarray(S, dtype=np.float64)
    ax = np.abs(x)[..., None]
    thr = _E2M1_MIDS * S[..., None]
    odd = (np.arange(7) % 2 == 1)
    up = np.where(odd, ax >= thr, ax > thr)
    mag = up.sum(axis=-1).astype(np.int64)
    mag = np.where(S == 0.0, 0, mag)
    sign = np.signbit(x).astype(np.int64) << 3
    return (sign | mag).astype(np.uint8)


def nvfp4_delayed_scale(amax_prev: float, headroom: float) -> np.float32:
    """Per-tensor scale from an earlier amax (README section 5.5, delayed
    amax): the amax found while quantizing one step, times a headroom,
    serves as the scale amax of the next step, so no pass over the tensor
    precedes its quantization.

    Reading (the page gives no formula): s_t is the NVFP4 tensor scale of the
    value headroom * amax_prev, computed as
    fp32_RNE(fp64(fp64(headroom * amax_prev) / 2688)), the same operation
    order on every side. Both inputs are fp32 quantities (an amax is kept as
    fp32 in the scale trailer, and the headroom is an fp32 argument), so they
    are rounded to fp32 first. With headroom 1 and amax_prev the tensor's own
    amax this is nvfp4_tensor_scale(amax).
    """
    h = np.float64(np.float32(headroom))
    a = np.float64(np.float32(amax_prev))
    return np.float32((h * a) / 2688.0)


def _quantize_nvfp4(x: np.ndarray, k_pad: int, s_t: np.float32):
    bs = 16
    blocks = _blocks(x, bs, k_pad)
    bamax = np.abs(blocks).max(axis=2)
    scales = nvfp4_block_bytes(bamax, s_t)
    S = F.e4m3_decode(scales) * np.float64(s_t)          # exact
    codes = nvfp4_element_codes(blocks, np.repeat(S[:, :, None], bs, axis=2))
    return codes.reshape(x.shape[0], k_pad), scales, s_t


def quantize(bits: np.ndarray, fmt: str, axis: str = "row", s_t=None) -> Quantized:
    """Quantize a bf16 tensor X [R, C] (given as uint16 bit patterns).

    axis="row": blocks run along C; stored operand is [R, round_up(C,128)].
    axis="col": blocks run along R; stored operand is X^T: [C, round_up(R,128)].
    NVFP4: s_t=None derives the tensor scale from X's own amax; a given s_t
    (e.g. nvfp4_delayed_scale) is used as is. The recorded amax is X's own
    either way.
    """
    if fmt not in FORMATS:
        raise ValueError(f"unknown format {fmt!r}")
    t = _view(bits, axis)
    x = F.bf16_to_f64(t)
    rows, length = x.shape
    k_pad = round_up(length, K_ALIGN)
    if fmt == "nvfp4":
        tensor_amax = float(np.abs(x).max()) if x.size else 0.0
        st = nvfp4_tensor_scale(tensor_amax) if s_t is None else np.float32(s_t)
        codes, scales, s_t = _quantize_nvfp4(x, k_pad, st)
        return Quantized(fmt, rows, length, k_pad, codes, scales,
                         s_t=s_t, amax=np.float32(tensor_amax))
    codes, scales = _quantize_mx(x, fmt, k_pad)
    return Quantized(fmt, rows, length, k_pad, codes, scales)


def quantize_dual(bits: np.ndarray, fmt: str, amax_prev=None, headroom: float = 32.0):
    """Both copies a training step needs (README section 5.5: one read of
    X, the row copy and the transposed copy written together): the
    quantization along axis "row" and along axis "col". For NVFP4 both use
    one tensor scale: X's own (amax_prev None) or the delayed scale
    nvfp4_delayed_scale(amax_prev, headroom)."""
    s_t = None
    if fmt == "nvfp4" and amax_prev is not None:
        s_t = nvfp4_delayed_scale(amax_prev, headroom)
    return quantize(bits, fmt, "row", s_t), quantize(bits, fmt, "col", s_t)


def codes_bytes(rows: int, cols: int, fmt: str, axis: str) -> int:
    """Bytes of the stored codes for X [rows, cols] quantized along `axis`."""
    r, length = (rows, cols) if axis == "row" else (cols, rows)
    k_pad = round_up(length, K_ALIGN)
    return r * (k_pad if fmt == "mxfp8" else k_pad // 2)


def scales_bytes(rows: int, cols: int, fmt: str, axis: str) -> int:
    """Bytes of the stored scale buffer (with the NVFP4 trailer)."""
    r, length = (rows, cols) if axis == "row" else (cols, rows)
    k_pad = round_up(length, K_ALIGN)
    n = r * (k_pad // block_size(fmt))
    if fmt == "nvfp4":
        return round_up(n, 16) + 16
    return n


# ------------------------------------------------------------------ stochastic rounding
#
# README section 5.3 (the P3 recipe: dgrad / wgrad in NVFP4 with gradients
# dY rounded stochastically) and section 5.5 (no hardware stochastic
# rounding, so it is done in software with Philox): the random numbers come
# from a counter-based generator, so that every element's draw is a pure
# function of (seed, element position) and any implementation that follows
# the same definition reproduces the codes bit for bit.
#
# Readings (the page names the method and the generator, not the details):
#   * generator: Philox4x64 with 10 rounds (Salmon, Moraes, Dror, Shaw,
#     "Parallel random numbers: as easy as 1, 2, 3", SC 2011), key = the
#     two 64-bit seed words, counter = (q, 0, 0, 0) for block q of eight
#     elements; element i = r * cols + c of the logical X [rows, cols] takes
#     32 bits of output word (i mod 8) // 2: the low half if i is even, the
#     high half if odd. The draw of an element does not depend on the axis.
#   * block scale bytes and s_t are exactly those of round-to-nearest.
#   * element: S32 = fp32(dec(byte) * s_t), y = fp32(|x| / S32) (IEEE,
#     round to nearest even); y >= 6 gives code 6 (saturation); otherwise
#     lo <= y < hi are neighbouring E2M1 grid values, frac = (y - lo) /
#     (hi - lo) (exact in fp32: Sterbenz for lo >= 0.5, and hi - lo is 0.5,
#     1 or 2), and the code is hi iff u < ceil(frac * 2^32), u the element's
#     32-bit draw; else lo. S32 == 0 gives signed zeros. The sign is x's.
#   These fp32 steps are the kernel's precision, fixed here so both sides
#   take the same integer decision.

_M64 = (1 << 64) - 1
_PHILOX_M = (np.uint64(0xD2E7470EE14C6C93), np.uint64(0xCA5A826395121157))
_PHILOX_W = (np.uint64(0x9E3779B97F4A7C15), np.uint64(0xBB67AE8584CAA73B))


def _mulhilo64(a: np.ndarray, b: np.uint64):
    """(high, low) 64-bit halves of the 128-bit products a * b (uint64)."""
    m32 = np.uint64(0xFFFFFFFF)
    s32 = np.uint64(32)
    a_lo, a_hi = a & m32, a >> s32
    b_lo, b_hi = b & m32, b >> s32
    ll, lh, hl, hh = a_lo * b_lo, a_lo * b_hi, a_hi * b_lo, a_hi * b_hi
    mid = (ll >> s32) + (lh & m32) + (hl & m32)
    hi = hh + (lh >> s32) + (hl >> s32) + (mid >> s32)
    return hi, a * b


def philox4x64(counters: np.ndarray, key) -> np.ndarray:
    """Philox4x64-10 of each row of counters [N, 4] (uint64) under the key
    (k0, k1): ten rounds of the four-word round function (two 64x64 -> 128
    multiplies whose high halves are xored into the other words together
    with the round key), the key bumped by the Weyl constants between
    rounds. Returns [N, 4] uint64."""
    c = np.array(counters, dtype=np.uint64).reshape(-1, 4)
    c0, c1, c2, c3 = (c[:, i].copy() for i in range(4))
    k0, k1 = np.uint64(key[0]), np.uint64(key[1])
    with np.errstate(over="ignore"):
        for _ in range(10):
            hi0, lo0 = _mulhilo64(c0, _PHILOX_M[0])
            hi1, lo1 = _mulhilo64(c2, _PHILOX_M[1])
            c0, c1, c2, c3 = hi1 ^ c1 ^ k0, lo1, hi0 ^ c3 ^ k1, lo0
            k0 = np.uint64((int(k0) + int(_PHILOX_W[0])) & _M64)
            k1 = np.uint64((int(k1) + int(_PHILOX_W[1])) & _M64)
    return np.stack([c0, c1, c2, c3], axis=1)


def sr_draws(rows: int, cols: int, seed) -> np.ndarray:
    """The 32-bit draw of every element of X [rows, cols] (uint32 [rows, cols])."""
    n = rows * cols
    nq = (n + 7) // 8
    ctr = np.zeros((nq, 4), dtype=np.uint64)
    ctr[:, 0] = np.arange(nq, dtype=np.uint64)
    words = philox4x64(ctr, seed)                              # [nq, 4]
    halves = np.empty((nq, 8), dtype=np.uint32)
    halves[:, 0::2] = (words & np.uint64(0xFFFFFFFF)).astype(np.uint32)
    halves[:, 1::2] = (words >> np.uint64(32)).astype(np.uint32)
    return halves.reshape(-1)[:n].reshape(rows, cols)


def nvfp4_element_codes_sr(x: np.ndarray, S32: np.ndarray, u: np.ndarray) -> np.ndarray:
    """E2M1 codes of x / S32 rounded stochastically with the draws u (the
    fp32 steps of the reading above); sign copied from x."""
    x = np.asarray(x, dtype=np.float64)
    S32 = np.asarray(S32, dtype=np.float32)
    a = np.abs(x).astype(np.float32)                           # exact: x is bf16
    with np.errstate(divide="ignore", invalid="ignore", over="ignore"):
        y = np.where(S32 > 0, a / np.where(S32 > 0, S32, np.float32(1)), np.float32(0)).astype(np.float32)
    grid = F.E2M1_GRID.astype(np.float32)                     # 0, .5, 1, 1.5, 2, 3, 4, 6
    lo_i = np.clip(np.searchsorted(grid, y, side="right") - 1, 0, 7)
    sat = y >= np.float32(6.0)
    hi_i = np.minimum(lo_i + 1, 7)
    lo, hi = grid[lo_i], grid[hi_i]
    span = np.where(sat, np.float32(1), hi - lo).astype(np.float32)
    frac = ((y - lo) / span).astype(np.float32)                # exact (see the reading)
    T = np.ceil(frac.astype(np.float64) * 4294967296.0)
    up = (~sat) & (np.asarray(u, dtype=np.float64) < T)
    mag = np.where(sat, 7, np.where(up, hi_i, lo_i)).astype(np.int64)
    mag = np.where(S32 > 0, mag, 0)
    sign = np.signbit(x).astype(np.int64) << 3
    return (sign | mag).astype(np.uint8)


def quantize_sr(bits: np.ndarray, axis: str, seed, s_t=None, draws=None) -> Quantized:
    """NVFP4 quantization of X along `axis` with stochastically rounded
    elements (block scales and s_t as quantize()); seed = (k0, k1). `draws`
    may pass sr_draws(rows, cols, seed) computed once for both copies."""
    rows0, cols0 = np.asarray(bits).shape
    if draws is None:
        draws = sr_draws(rows0, cols0, seed)
    t = _view(bits, axis)
    u = draws if axis == "row" else np.ascontiguousarray(draws.T)
    x = F.bf16_to_f64(t)
    rows, length = x.shape
    k_pad = round_up(length, K_ALIGN)
    tensor_amax = float(np.abs(x).max()) if x.size else 0.0
    st = nvfp4_tensor_scale(tensor_amax) if s_t is None else np.float32(s_t)
    bs = 16
    blocks = _blocks(x, bs, k_pad)
    bamax = np.abs(blocks).max(axis=2)
    scales = nvfp4_block_bytes(bamax, st)
    S32 = (F.e4m3_decode(scales).astype(np.float32) * np.float32(st)).astype(np.float32)
    ublocks = np.zeros((rows, k_pad), dtype=np.uint32)
    ublocks[:, :length] = u
    codes = nvfp4_element_codes_sr(blocks, np.repeat(S32[:, :, None], bs, axis=2),
                                   ublocks.reshape(rows, k_pad // bs, bs))
    return Quantized("nvfp4", rows, length, k_pad, codes.reshape(rows, k_pad), scales,
                     s_t=st, amax=np.float32(tensor_amax))


def quantize_dual_sr(bits: np.ndarray, seed, amax_prev=None, headroom: float = 32.0):
    """Row and column NVFP4 copies with stochastic rounding, one tensor scale
    (X's own, or the delayed one) and one draw per element shared by both."""
    s_t = None if amax_prev is None else nvfp4_delayed_scale(amax_prev, headroom)
    draws = sr_draws(*np.asarray(bits).shape, seed)
    return quantize_sr(bits, "row", seed, s_t, draws), quantize_sr(bits, "col", seed, s_t, draws)
