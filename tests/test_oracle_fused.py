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
