"""Pins for oracle/formats.py against definitions written independently here.

Every reference below decodes bit fields with exact Fractions and rounds by
brute-force nearest search, so a wrong bias, a dropped subnormal, a wrong
tie rule or a wrong saturation in the oracle fails a test.
"""
import bisect
import math
import os
from fractions import Fraction

import numpy as np
import pytest

from oracle import formats as F

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


# ------------------------------------------------------------ references

def frac_bf16(bits: int) -> Fraction:
    s = -1 if bits >> 15 else 1
    e = (bits >> 7) & 0xFF
    m = bits & 0x7F
    if e == 0:
        return s * Fraction(m, 128) * Fraction(2) ** -126
    return s * (1 + Fraction(m, 128)) * Fraction(2) ** (e - 127)


def frac_e4m3(code: int):
    s = -1 if code & 0x80 else 1
    e = (code >> 3) & 0xF
    m = code & 7
    if (code & 0x7F) == 0x7F:
        return None
    if e == 0:
        return s * Fraction(m, 8) * Fraction(2) ** -6
    return s * (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)


def frac_e2m1(code: int) -> Fraction:
    s = -1 if code & 8 else 1
    e = (code >> 1) & 3
    m = code & 1
    if e == 0:
        return s * Fraction(m, 2)
    return s * (1 + Fraction(m, 2)) * Fraction(2) ** (e - 1)


E4M3_POS = [(frac_e4m3(c), c) for c in range(0x7F)]       # magnitudes 0..448
E2M1_POS = [(frac_e2m1(c), c) for c in range(8)]


def ref_rne(v: Fraction, table) -> int:
    """Nearest grid value to |v| (ties: even code), saturating; sign copied."""
    sign = v < 0
    a = abs(v)
    vals = [t[0] for t in table]
    if a >= vals[-1]:
        mag = table[-1][1]
    else:
        i = bisect.bisect_right(vals, a)    # vals[i-1] <= a < vals[i]
        lo, hi = table[i - 1], table[i]
        dlo, dhi = a - lo[0], hi[0] - a
        if dlo < dhi:
            mag = lo[1]
        elif dhi < dlo:
            mag = hi[1]
        else:
            mag = lo[1] if lo[1] % 2 == 0 else hi[1]
    return mag


# ------------------------------------------------------------ golden facts

def _read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if line and not line.startswith("#"):
                rows.append(line.split())
    return rows


def test_golden_bf16_row_of_format_table():
    """bf16 = 8 exponent + 7 mantissa bits, eps 7.8e-3, max 3.4e38 (blog section 2)."""
    row = {r[0]: r for r in _read_golden("float_formats.txt")}["BF16"]
    exp_bits, man_bits, eps, mx = int(row[1]), int(row[2]), float(row[3]), float(row[4])
    one = 0x3F80
    eps_oracle = F.bf16_to_f64(np.array([one + 1]))[0] - 1.0
    assert eps_oracle == 2.0 ** -man_bits
    assert f"{eps_oracle:.1e}" == f"{eps:.1e}"
    mx_oracle = F.bf16_to_f64(np.array([0x7F7F]))[0]
    assert f"{mx_oracle:.1e}" == f"{mx:.1e}"
    # exponent field width: 0x7F80 is the first non-finite pattern
    assert not np.isfinite(F.bf16_to_f64(np.array([0x7F80]))[0])
    assert (0x7F80 >> man_bits) == (1 << exp_bits) - 1


def test_golden_e4m3_max_448():
    """The largest E4M3 value is 448 (blog section 5.4)."""
    row = {r[0]: r for r in _read_golden("float_formats.txt")}["E4M3"]
    assert F.E4M3_GRID.max() == float(row[4]) == F.E4M3_MAX
    assert F.e4m3_encode(np.array([1e9]))[0] == 0x7E
    assert F.e4m3_decode(np.array([0x7E]))[0] == 448.0


# ------------------------------------------------------------ bf16

def test_bf16_decode_all_patterns():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    got = F.bf16_to_f64(bits)
    for b in range(65536):
        if ((b >> 7) & 0xFF) == 0xFF:
            assert not np.isfinite(got[b])
            continue
        assert Fraction(float(got[b])) == frac_bf16(b), hex(b)


def ref_bf16_round(v: Fraction) -> Fraction:
    """RNE of an exact rational to the bf16 grid (finite range only)."""
    if v == 0:
        return Fraction(0)
    s = -1 if v < 0 else 1
    a = abs(v)
    e = math.floor(math.log2(a))
    while Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    q = Fraction(2) ** max(e - 7, -133)
    n = a / q
    fl = math.floor(n)
    r = n - fl
    if r > Fraction(1, 2) or (r == Fraction(1, 2) and fl % 2 == 1):
        fl += 1
    return s * fl * q


def test_bf16_round_from_f64_matches_exact_rounding():
    rng = np.random.default_rng(7)
    x = np.concatenate([
        rng.standard_normal(3000) * 10.0 ** rng.integers(-30, 30, 3000),
        rng.standard_normal(200) * 2.0 ** -130,          # bf16 subnormal range
    ])
    # exact midpoints between bf16 neighbours and their float64 neighbours
    b = F.bf16_to_f64(rng.integers(0x0080, 0x7F00, 500).astype(np.uint16))
    ulp = np.ldexp(1.0, np.frexp(b)[1] - 8)
    mids = b + ulp / 2
    x = np.concatenate([x, mids, np.nextafter(mids, np.inf), np.nextafter(mids, -np.inf), -mids])
    got = F.f64_to_bf16_rne(x)
    for xi, gi in zip(x, got):
        assert Fraction(float(gi)) == ref_bf16_round(Fraction(float(xi))), xi


def test_bf16_bits_roundtrip():
    bits = np.arange(0, 0x7F80, 3, dtype=np.uint32).astype(np.uint16)
    assert np.array_equal(F.f64_to_bf16_bits(F.bf16_to_f64(bits)), bits)


# ------------------------------------------------------------ E4M3

def test_e4m3_decode_table_vs_bitfields():
    got = F.e4m3_decode(np.arange(256, dtype=np.uint8))
    for c in range(256):
        ref = frac_e4m3(c)
        if ref is None:
            assert np.isnan(got[c])
        else:
            assert Fraction(float(got[c])) == ref, hex(c)


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], dtype=np.uint8)
    assert len(codes) == 254
    vals = F.e4m3_decode(codes)
    vals = np.where(codes == 0x80, -0.0, vals)
    back = F.e4m3_encode(vals)
    assert np.array_equal(back, codes)


def test_e4m3_midpoints_and_neighbours():
    g = F.E4M3_GRID
    for i in range(len(g) - 1):
        mid = (g[i] + g[i + 1]) / 2
        even = i if i % 2 == 0 else i + 1
        assert F.e4m3_encode(np.array([mid]))[0] == even
        assert F.e4m3_encode(np.array([-mid]))[0] == 0x80 | even
        assert F.e4m3_encode(np.array([np.nextafter(mid, 0)]))[0] == i
        assert F.e4m3_encode(np.array([np.nextafter(mid, np.inf)]))[0] == i + 1


def test_e4m3_saturation():
    for v in [448.0, 448.0 + 1e-9, 464.0, 480.0, 1e30]:
        assert F.e4m3_encode(np.array([v]))[0] == 0x7E
        assert F.e4m3_encode(np.array([-v]))[0] == 0xFE


def test_e4m3_encode_exhaustive_bf16_significands():
    """Every bf16 significand in every binade 2^-20 .. 2^12, both signs."""
    mants = np.arange(128)
    vals = []
    for t in range(-20, 13):
        vals.append((1 + mants / 128.0) * 2.0 ** t)
    v = np.concatenate(vals + [np.array([0.0, -0.0])])
    v = np.concatenate([v, -v])
    got = F.e4m3_encode(v)
    for x, c in zip(v, got):
        ref = ref_rne(Fraction(float(x)), E4M3_POS) | (0x80 if math.copysign(1, x) < 0 else 0)
        assert c == ref, (x, c, ref)


# ------------------------------------------------------------ E2M1

def test_e2m1_decode_table_vs_bitfields():
    got = F.e2m1_decode(np.arange(16, dtype=np.uint8))
    for c in range(16):
        assert Fraction(float(got[c])) == frac_e2m1(c)
    assert list(F.E2M1_GRID) == [0, 0.5, 1, 1.5, 2, 3, 4, 6]


def test_e2m1_roundtrip_all_codes():
    codes = np.arange(16, dtype=np.uint8)
    vals = F.e2m1_decode(codes)
    vals = np.where(codes == 8, -0.0, vals)
    assert np.array_equal(F.e2m1_encode(vals), codes)


def test_e2m1_ties_to_even():
    ties = {0.25: 0.0, 0.75: 1.0, 1.25: 1.0, 1.75: 2.0, 2.5: 2.0, 3.5: 4.0, 5.0: 4.0}
    for v, want in ties.items():
        got = F.e2m1_decode(F.e2m1_encode(np.array([v, -v])))
        assert got[0] == want and got[1] == -want


def test_e2m1_encode_exhaustive_bf16_significands():
    mants = np.arange(128)
    v = np.concatenate([(1 + mants / 128.0) * 2.0 ** t for t in range(-8, 6)] + [np.array([0.0, -0.0])])
    v = np.concatenate([v, -v])
    got = F.e2m1_encode(v)
    for x, c in zip(v, got):
        ref = ref_rne(Fraction(float(x)), E2M1_POS) | (8 if math.copysign(1, x) < 0 else 0)
        assert c == ref, (x, c, ref)


def test_e2m1_saturation():
    assert F.e2m1_encode(np.array([6.0, 7.0, 1e9]))[0] == 7
    assert np.all(F.e2m1_encode(np.array([6.0, 7.0, 1e9])) == 7)
    assert np.all(F.e2m1_encode(np.array([-6.0, -7.0, -1e9])) == 15)


def test_negative_zero_codes():
    assert F.e4m3_encode(np.array([-0.0]))[0] == 0x80
    assert F.e4m3_encode(np.array([-1e-6]))[0] == 0x80
    assert F.e2m1_encode(np.array([-0.0, -0.2]))[0] == 8
    assert F.e2m1_encode(np.array([-0.2]))[0] == 8


def test_floor_log2_exact():
    for k in range(-140, 130):
        for m in (1.0, 1.5, 1.9999999):
            a = m * 2.0 ** k
            if a == 0 or not np.isfinite(a):
                continue
            assert F.floor_log2(a) == k
