"""Pins of oracle.layernorm (LayerNorm fused with quantization), each from
something other than the oracle's own formula: the two-element closed form,
the library LayerNorm, invariances, the normalized moments, the affine
split, constant rows, planted mistakes, and the acceptance check against an
fp32 evaluation of the kernel's arithmetic."""
import numpy as np
import pytest
import torch

from oracle import formats as F
from oracle import fused as FU
from oracle import layernorm as L
from oracle import quantize as Q


def rows(r, c, seed, offset=0.0, scale=1.0):
    x = np.random.default_rng(seed).standard_normal((r, c)) * scale + offset
    return x.astype(np.float32)


def test_two_elements_closed_form():
    """C = 2: mu = (a + b) / 2 and var = ((a - b) / 2)^2, so
    y_0 = h / sqrt(h^2 + eps) with h = (a - b) / 2, and y_1 = -y_0."""
    ab = np.array([[3.0, 1.0], [-2.5, 4.0], [7.0, 7.0], [1e-3, -1e-3]], dtype=np.float32)
    eps = 1e-6
    y = L.layernorm(ab, np.ones(2, np.float32), np.zeros(2, np.float32), eps)
    for (a, b), (y0, y1) in zip(ab.astype(np.float64), y):
        h = (a - b) / 2
        want = h / np.sqrt(h * h + eps)
        assert y0 == pytest.approx(want, rel=1e-14, abs=1e-300)
        assert y1 == pytest.approx(-want, rel=1e-14, abs=1e-300)


@pytest.mark.parametrize("c, eps", [(1024, 1e-6), (300, 1e-5), (4096, 1e-6)])
def test_matches_library_layer_norm(c, eps):
    x = rows(6, c, seed=c, offset=0.5, scale=2.0)
    rng = np.random.default_rng(c + 1)
    g = rng.standard_normal(c).astype(np.float32)
    b = rng.standard_normal(c).astype(np.float32)
    ref = torch.nn.functional.layer_norm(torch.from_numpy(x.astype(np.float64)), (c,),
                                         torch.from_numpy(g.astype(np.float64)),
                                         torch.from_numpy(b.astype(np.float64)), eps).numpy()
    np.testing.assert_allclose(L.layernorm(x, g, b, eps), ref, rtol=1e-12, atol=1e-12)


def test_shift_and_scale_invariance():
    """Shifting a row by a constant leaves LayerNorm unchanged; scaling it
    by a power of two too when eps = 0 (small integers keep both exact)."""
    x = np.random.default_rng(3).integers(-50, 50, (5, 96)).astype(np.float32)
    g = np.random.default_rng(4).standard_normal(96).astype(np.float32)
    b = np.random.default_rng(5).standard_normal(96).astype(np.float32)
    base = L.layernorm(x, g, b, 1e-6)
    np.testing.assert_allclose(L.layernorm(x + np.float32(1024), g, b, 1e-6), base, rtol=0, atol=1e-13)
    base0 = L.layernorm(x, g, b, 0.0)
    np.testing.assert_allclose(L.layernorm(x * np.float32(8), g, b, 0.0), base0, rtol=0, atol=1e-13)


def test_normalized_moments():
    """gamma = 1, beta = 0: every row has mean 0 and mean square
    var / (var + eps)."""
    x = rows(7, 512, seed=9, offset=3.0, scale=0.01)
    eps = 1e-5
    y = L.layernorm(x, np.ones(512, np.float32), np.zeros(512, np.float32), eps)
    xd = x.astype(np.float64)
    var = xd.var(axis=1)
    np.testing.assert_allclose(y.mean(axis=1), 0.0, atol=1e-12)
    np.testing.assert_allclose((y * y).mean(axis=1), var / (var + eps), rtol=1e-12)


def test_affine_split_and_constant_rows():
    x = rows(4, 128, seed=11)
    x[2] = np.float32(2.75)                     # a constant row: var = 0
    rng = np.random.default_rng(12)
    g = rng.standard_normal(128).astype(np.float32)
    b = rng.standard_normal(128).astype(np.float32)
    y = L.layernorm(x, g, b, 1e-6)
    plain = L.layernorm(x, np.ones(128, np.float32), np.zeros(128, np.float32), 1e-6)
    np.testing.assert_allclose(y, plain * g.astype(np.float64) + b.astype(np.float64), rtol=1e-14, atol=1e-14)
    assert np.array_equal(y[2], b.astype(np.float64))


@pytest.mark.parametrize("mistake", ["unbiased variance", "eps outside the root", "gamma and beta swapped"])
def test_planted_mistakes_fail_a_pin(monkeypatch, mistake):
    """Each plausible slip in the oracle is caught by one of the pins above."""
    orig_stats = L._stats

    if mistake == "unbiased variance":
        def bad_stats(x, eps):
            x = np.asarray(x, np.float64)
            mu = x.mean(axis=1, keepdims=True)
            var = ((x - mu) ** 2).sum(axis=1, keepdims=True) / (x.shape[1] - 1)
            return x, mu, var, 1.0 / np.sqrt(var + eps)
        monkeypatch.setattr(L, "_stats", bad_stats)
    elif mistake == "eps outside the root":
        def bad_stats(x, eps):
            with np.errstate(divide="ignore"):
                x, mu, var, _ = orig_stats(x, 0.0)
            return x, mu, var, 1.0 / (np.sqrt(var) + eps)
        monkeypatch.setattr(L, "_stats", bad_stats)
    else:
        orig = L.layernorm
        monkeypatch.setattr(L, "layernorm", lambda x, g, b, eps: orig(x, b, g, eps))
    failed = 0
    for pin in (test_two_elements_closed_form, test_normalized_moments, test_affine_split_and_constant_rows,
                lambda: test_matches_library_layer_norm(300, 1e-5)):
        try:
            pin()
        except AssertionError:
            failed += 1
    assert failed >= 1, f"no pin catches: {mistake}"


def fp32_layernorm(x, g, b, eps):
    """LayerNorm in fp32 arithmetic with pairwise row sums (numpy float32),
    the kind of evaluation the kernel does, rounded to bf16."""
    x = np.asarray(x, np.float32)
    c = np.float32(x.shape[1])
    mu = x.sum(axis=1, dtype=np.float32, keepdims=True) / c
    d = (x - mu).astype(np.float32)
    var = (d * d).sum(axis=1, dtype=np.float32, keepdims=True) / c
    r = (np.float32(1) / np.sqrt(var + np.float32(eps))).astype(np.float32)
    y = (d * r).astype(np.float32) * g + b
    return F.f64_to_bf16_bits(y.astype(np.float64))


@pytest.mark.parametrize("fmt", ["mxfp8", "mxfp4"])
@pytest.mark.parametrize("offset", [0.0, 300.0])
def test_check_accepts_fp32_evaluation_and_rejects_mistakes(fmt, offset):
    """The acceptance check takes the exact reference and an fp32
    evaluation (also with a mean far above the spread, where the mean's
    rounding dominates), and rejects a code one step off and a scale byte
    one too large."""
    c = 1000
    x = rows(8, c, seed=21, offset=offset, scale=1.5)
    rng = np.random.default_rng(22)
    g = (1 + 0.1 * rng.standard_normal(c)).astype(np.float32)
    b = (0.1 * rng.standard_normal(c)).astype(np.float32)
    eps = 1e-6
    for q in (L.reference_codes(x, g, b, eps, fmt), Q.quantize(fp32_layernorm(x, g, b, eps), fmt, "row")):
        ok_c, ok_s = L.check_rows(q.codes, q.scales, x, g, b, eps, fmt)
        assert ok_c.all() and ok_s.all()
    q = L.reference_codes(x, g, b, eps, fmt)
    codes = q.codes.copy()
    i, j = 3, 517
    codes[i, j] = (codes[i, j] & 0x80) | min((codes[i, j] & 0x7F) + 1, 0x7E) if fmt == "mxfp8" else \
        (codes[i, j] & 0x8) | min((codes[i, j] & 0x7) + 1, 7)
    assert codes[i, j] != q.codes[i, j]
    ok_c, _ = L.check_rows(codes, q.scales, x, g, b, eps, fmt)
    assert not ok_c[i, j] and ok_c.sum() == ok_c.size - 1
    scales = q.scales.copy()
    scales[5, 7] += 1
    _, ok_s = L.check_rows(q.codes, scales, x, g, b, eps, fmt)
    assert not ok_s[5, 7] and ok_s.sum() == ok_s.size - 1


def test_padding_codes_must_be_zero():
    x = rows(2, 200, seed=31)
    g, b = np.ones(200, np.float32), np.zeros(200, np.float32)
    q = L.reference_codes(x, g, b, 1e-6, "mxfp8")
    assert q.codes.shape[1] == 256 and not q.codes[:, 200:].any()
    codes = q.codes.copy()
    codes[1, 230] = 0x01
    ok_c, _ = L.check_rows(codes, q.scales, x, g, b, 1e-6, "mxfp8")
    assert not ok_c[1, 230]
    assert FU.check_intervals  # the shared acceptance used above


def _enc(v, e, fmt):
    x = np.ldexp(np.asarray(v, dtype=np.float64), -e)
    return F.e4m3_encode(x) if fmt == "mxfp8" else F.e2m1_encode(x)


def test_scale_and_codes_must_come_from_one_choice():
    """A constant row (x = 40, so 1/sqrt(var + eps) = 1000 and the allowance
    2^-16 (r |mu| + |beta| + |y|) is about 0.61) with beta = 4 in column 0:
    y0 may be anything in about [3.39, 4.61], straddling MXFP4's binade
    boundary 4 = 2^emax. Block exponent 0 with every code taken from the
    intervals' low ends (y0 -> code 3) is explained by no single choice (a
    y0 that encodes to 3 is below 4, so the amax would give exponent -1),
    although each code and the exponent are possible on their own. The exact
    LayerNorm output (exponent 0, y0 = 4) is accepted."""
    fmt, cols, eps = "mxfp4", 64, 1e-6
    x = np.full((1, cols), 40.0, np.float32)
    g = np.ones(cols, np.float32)
    b = np.full(cols, 0.5, np.float32)
    b[0] = 4.0
    y, tol = L.tolerance(x, g, b, eps)
    lo, hi = F.f64_to_bf16_rne(y - tol), F.f64_to_bf16_rne(y + tol)
    assert lo[0, 0] < 3.5 and hi[0, 0] >= 4.0
    planted = np.zeros((1, 128), np.uint8)
    planted[0, :cols] = _enc(lo, 0, fmt)
    assert F.e2m1_decode(planted[0, 0]) == 3.0
    scales = np.array([[127, 0, 0, 0]], np.uint8)
    scales[0, 1] = L.reference_codes(x, g, b, eps, fmt).scales[0, 1]
    ok_c, ok_s = L.check_rows(planted, scales, x, g, b, eps, fmt)
    assert ok_c.all() and not ok_s[0, 0]
    q = L.reference_codes(x, g, b, eps, fmt)
    assert q.scales[0, 0] == 127
    ok_c, ok_s = L.check_rows(q.codes, q.scales, x, g, b, eps, fmt)
    assert ok_c.all() and ok_s.all()


def test_zero_codes_keep_the_sign():
    """Elements whose LayerNorm output is negative (interval entirely below
    zero) but rounds to zero at the block's exponent carry the negative-zero
    code; the positive zero there is rejected. MXFP4 only: for MXFP8 the
    allowance is wider than the values that round to zero, so every zero
    code's interval straddles zero and either sign is right."""
    fmt = "mxfp4"
    x = rows(16, 512, seed=41, scale=1.0)
    rng = np.random.default_rng(42)
    g = (1 + 0.1 * rng.standard_normal(512)).astype(np.float32)
    b = (0.05 * rng.standard_normal(512)).astype(np.float32)
    eps = 1e-6
    q = L.reference_codes(x, g, b, eps, fmt)
    y, tol = L.tolerance(x, g, b, eps)
    hi = F.f64_to_bf16_rne(y + tol)
    neg_zero = 0x80 if fmt == "mxfp8" else 0x8
    cand = np.argwhere((q.codes[:, :512] == neg_zero) & (hi < 0))
    assert len(cand) >= 5, len(cand)
    bad = q.codes.copy()
    r, c = cand[:, 0], cand[:, 1]
    bad[r, c] = 0
    ok_c, _ = L.check_rows(bad, q.scales, x, g, b, eps, fmt)
    assert not ok_c[r, c].any() and ok_c.sum() == ok_c.size - len(cand)
