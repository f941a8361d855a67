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
