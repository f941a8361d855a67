"""Pins of the fused fc1 -> GELU -> quantize oracle (oracle/fused.py): the
GELU against the normal CDF of a library and against identities, the
minimum, and the acceptance check against its own reference and against
planted mistakes."""
import numpy as np
import pytest
from scipy.stats import norm

from oracle import formats as F
from oracle import fused as FU
from oracle import quantize as Q


def test_gelu_is_x_times_the_normal_cdf():
    x = np.linspace(-12, 12, 4001)
    assert np.allclose(FU.gelu(x), x * norm.cdf(x), rtol=1e-13, atol=1e-300)


def test_gelu_identities():
    x = np.linspace(-30, 30, 6001)
    assert np.allclose(FU.gelu(x) - FU.gelu(-x), x, rtol=0, atol=1e-12)   # Phi(x) + Phi(-x) = 1
    assert FU.gelu(0.0) == 0.0
    big = np.array([10.0, 20.0, 38.0])
    assert np.array_equal(FU.gelu(big), big)                              # Phi(x) = 1 in float64
    assert np.all(FU.gelu(-big) <= 0) and np.all(FU.gelu(-big) > -1e-20)


def test_gelu_minimum():
    m = FU.GELU_ARGMIN
    assert -0.76 < m < -0.75
    assert FU._gelu_slope(m - 1e-6) < 0 < FU._gelu_slope(m + 1e-6)
    xs = np.linspace(-3, 1, 40001)
    assert FU.gelu(m) <= FU.gelu(xs).min() + 1e-15


def _rows(fmt, seed, rows=6, n=96):
    """bf16 pre-activations h with 8 significant bits (exact in bf16), and the
    reference output: with c = h and gemm_tol = 0 the only slack is the GELU
    allowance."""
    rng = np.random.default_rng(seed)
    h = rng.standard_normal((rows, n)) * 2.0
    h[0, :8] = [0.0, -0.7517, 5.0, -5.0, 1e-3, -1e-3, 12.0, -12.0]
    h_bits = F.f64_to_bf16_bits(h)
    hq = F.bf16_to_f64(h_bits)
    ref = FU.reference_codes(h_bits, fmt)
    codes = FU.unpack_codes(ref.packed_codes(), fmt)
    return hq, codes, ref.scales.copy()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_check_accepts_its_reference(fmt):
    hq, codes, scales = _rows(fmt, 1)
    ok_c, ok_s = FU.check_rows(codes, scales, hq, np.zeros_like(hq), fmt, hq.shape[1], gemm_tol=0.0)
    assert ok_c.all() and ok_s.all()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_check_rejects_planted_mistakes(fmt):
    hq, codes, scales = _rows(fmt, 2)
    n = hq.shape[1]
    z = np.zeros_like(hq)
    # a code moved one grid step (magnitude +1 on a non-saturated, nonzero code)
    bad = codes.copy()
    i = next(i for i in range(n) if 0 < (bad[3, i] & 0x7) < 6)
    bad[3, i] += 1
    ok_c, _ = FU.check_rows(bad, scales, hq, z, fmt, n, 0.0)
    assert not ok_c[3, i]
    # a sign flipped
    bad = codes.copy()
    j = next(j for j in range(n) if (bad[2, j] & 0x7) != 0)
    bad[2, j] ^= 0x80 if fmt == "mxfp8" else 0x8
    ok_c, _ = FU.check_rows(bad, scales, hq, z, fmt, n, 0.0)
    assert not ok_c[2, j]
    # a scale byte one too large
    sc = scales.copy()
    sc[1, 0] += 1
    _, ok_s = FU.check_rows(codes, sc, hq, z, fmt, n, 0.0)
    assert not ok_s[1, 0]
    # no GELU at all: quantize(h) instead of quantize(GELU(h))
    noact = Q.quantize(F.f64_to_bf16_bits(hq), fmt, "row")
    ok_c, ok_s = FU.check_rows(FU.unpack_codes(noact.packed_codes(), fmt), noact.scales, hq, z, fmt, n, 0.0)
    assert ok_c.mean() < 0.8
    # nonzero padding codes
    bad = codes.copy()
    bad[0, n] = 1
    ok_c, _ = FU.check_rows(bad, scales, hq, z, fmt, n, 0.0)
    assert not ok_c[0, n]


def test_check_gemm_slack_widens_the_intervals():
    """A GEMM bound of several bf16 ulps admits the neighbouring codes."""
    hq, codes, scales = _rows("mxfp8", 3)
    s = np.abs(hq) * 64.0                 # TOL * S = |h| / 64, several bf16 ulps
    ok_c, ok_s = FU.check_rows(codes, scales, hq, s, "mxfp8", hq.shape[1])
    assert ok_c.all() and ok_s.all()


# ---------------------------------------------------------------- joint acceptance

def _enc(v, e, fmt):
    """Codes of v at shared exponent e (the oracle's RNE encoders)."""
    x = np.ldexp(np.asarray(v, dtype=np.float64), -e)
    return F.e4m3_encode(x) if fmt == "mxfp8" else F.e2m1_encode(x)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_scale_and_codes_must_come_from_one_choice(fmt):
    """Element 0 may be anything in [lo0, hi0], an interval that straddles
    the binade boundary 2^emax of block exponent 0; the others are small.
    Exponent 0 is possible (element 0 at its high end) and so is -1 (at its
    low end). An output with exponent 0 but every code encoded from the
    interval's low ends is explained by no single choice: its element-0 code
    can only come from values below 2^emax, so the block amax would give
    exponent -1. The per-element view (scale within the exponents of the
    smallest and largest possible amax, each code within its interval's end
    codes) accepts it; the joint check must not."""
    emax = F.E4M3_EMAX if fmt == "mxfp8" else F.E2M1_EMAX
    top = 2.0 ** emax
    lo0, hi0 = (200.0, 260.0) if fmt == "mxfp8" else (3.25, 4.5)
    assert lo0 < top <= hi0
    n = 32
    g_lo = np.full((1, n), 1.0)
    g_hi = np.full((1, n), 1.5)
    g_lo[0, 0], g_hi[0, 0] = lo0, hi0
    # the planted output: exponent 0, codes from the low ends
    planted = _enc(g_lo, 0, fmt)
    assert F.e4m3_decode(planted[0, 0]) < top if fmt == "mxfp8" else F.e2m1_decode(planted[0, 0]) < top
    ok_c, ok_s = FU.check_intervals(planted, np.array([[127]]), g_lo, g_hi, fmt, n)
    assert ok_c.all()                      # every code alone is possible at exponent 0
    assert not ok_s[0, 0]                  # but not together with that exponent
    # consistent outputs: exponent 0 with element 0 at its high end, exponent -1 at the low end
    for e, pick in ((0, g_hi), (-1, g_lo)):
        codes = _enc(pick, e, fmt)
        ok_c, ok_s = FU.check_intervals(codes, np.array([[127 + e]]), g_lo, g_hi, fmt, n)
        assert ok_c.all() and ok_s.all(), (e, ok_c, ok_s)


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_zero_codes_keep_the_sign(fmt):
    """A value that rounds to zero at the block's exponent keeps its sign in
    the code (negative-zero code for a negative value): an interval entirely
    below zero admits only the negative zero, one entirely above only the
    positive zero, one that straddles zero both. -0 == +0 as numbers, so a
    check on decoded values cannot see this."""
    big, tiny = (300.0, 3e-4) if fmt == "mxfp8" else (6.0, 0.1)
    neg_zero = 0x80 if fmt == "mxfp8" else 0x8
    n = 32
    g_lo = np.full((1, n), 1.0)
    g_hi = np.full((1, n), 1.0)
    g_lo[0, 0] = g_hi[0, 0] = big                        # exponent 0
    g_lo[0, 1], g_hi[0, 1] = -2 * tiny, -tiny            # negative: -0 only
    g_lo[0, 2], g_hi[0, 2] = tiny, 2 * tiny              # positive: +0 only
    g_lo[0, 3], g_hi[0, 3] = -tiny, tiny                 # straddles zero: either
    g_lo[0, 4], g_hi[0, 4] = -0.0, -0.0                  # exactly -0: -0 only
    lo_b = F.f64_to_bf16_rne(g_lo)
    hi_b = F.f64_to_bf16_rne(g_hi)
    codes = _enc(lo_b, 0, fmt)
    assert codes[0, 1] == neg_zero and codes[0, 2] == 0 and codes[0, 4] == neg_zero
    sc = np.array([[127]])
    ok_c, ok_s = FU.check_intervals(codes, sc, lo_b, hi_b, fmt, n)
    assert ok_c.all() and ok_s.all()
    for i, flipped in ((1, 0), (2, neg_zero), (4, 0)):
        bad = codes.copy()
        bad[0, i] = flipped
        ok_c, _ = FU.check_intervals(bad, sc, lo_b, hi_b, fmt, n)
        assert not ok_c[0, i] and ok_c.sum() == n - 1, i
    for z in (0, neg_zero):
        other = codes.copy()
        other[0, 3] = z
        ok_c, _ = FU.check_intervals(other, sc, lo_b, hi_b, fmt, n)
        assert ok_c.all()


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
def test_gelu_of_negative_h_gives_negative_zero_codes(fmt):
    """GELU(h) has the sign of h. For h far below zero GELU(h) is a tiny
    negative number (-0 in bf16 from h = -14 on), so its code at the block's
    exponent is the negative zero; a positive-zero code there is a
    mistake the check must catch (the fused kernel's fp32 GELU must not
    turn these into +0)."""
    h = np.zeros((1, 64))
    h[0, 0] = 8.0                                   # the block amax
    h[0, 1:16] = -np.array([4, 6, 8, 10, 12, 13, 14, 16, 20, 30, 100, 1e3, 1e10, 1e30, 3e38])
    h[0, 16:32] = np.linspace(0.5, 3.0, 16)
    h[0, 32:] = -np.geomspace(14, 1e38, 32)          # a whole block of negatives only
    hq = F.bf16_to_f64(F.f64_to_bf16_bits(h))
    ref = FU.reference_codes(F.f64_to_bf16_bits(h), fmt)
    codes = FU.unpack_codes(ref.packed_codes(), fmt)
    neg_zero = 0x80 if fmt == "mxfp8" else 0x8
    z = np.zeros_like(hq)
    ok_c, ok_s = FU.check_rows(codes, ref.scales, hq, z, fmt, 64, 0.0)
    assert ok_c.all() and ok_s.all()
    zeros = np.flatnonzero(codes[0, :64] == neg_zero)
    assert zeros.size >= 10
    bad = codes.copy()
    bad[0, zeros] = 0
    ok_c, _ = FU.check_rows(bad, ref.scales, hq, z, fmt, 64, 0.0)
    assert not ok_c[0, zeros].any()


def test_gelu_underflow_allowance_covers_a_flushed_tail():
    """GELU_ABS = 2^-126 covers an exp2 factor flushed to zero: that happens
    only where exp(-z^2/2) < 2^-126, and there |GELU| = z Q(z) is below
    phi(z) = exp(-z^2/2) / sqrt(2 pi) (Q(z) < phi(z) / z, checked against the
    library's normal tail), hence below 2^-127."""
    from scipy.stats import norm
    z = np.linspace(0.05, 37.0, 20000)
    assert np.all(z * norm.sf(z) < norm.pdf(z))
    zf = np.sqrt(2 * 126 * np.log(2))               # exp(-z^2/2) = 2^-126 here
    zz = np.linspace(zf, zf + 10, 2000)
    assert np.all(zz * norm.sf(zz) < 2.0 ** -127)
    assert FU.GELU_ABS == 2.0 ** -126
