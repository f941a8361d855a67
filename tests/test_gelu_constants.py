"""The fused epilogue's fp32 GELU (gelu_f32 in csrc/gemm_mx.hip) is tied to
its derivation (csrc/gelu_fit.py) and to the accuracy the C header states:
the constants are read out of the kernel source, the tail polynomial is
evaluated the way the kernel does (fp32 Horner with fused multiply-adds) and
compared with the normal tail of a library, and a fit at the kernel's p
reproduces the kernel's coefficients."""
import importlib.util
import os
import re

import numpy as np
from scipy.special import erfcx

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "block_scaled_precision_mx_amd", "csrc")


def kernel_constants():
    """(p, [c0 .. c7]) of gelu_f32 as written in gemm_mx.hip."""
    src = open(os.path.join(CSRC, "gemm_mx.hip")).read()
    body = src[src.index("float gelu_f32(float h)"):]
    body = body[:body.index("\n}\n")]
    p = float(re.search(r"rcpf\(fmaf\(([-0-9.e]+)f, z, 1\.0f\)\)", body).group(1))
    top = float(re.search(r"float r = ([-0-9.e]+)f;", body).group(1))
    rest = [float(v) for v in re.findall(r"r = fmaf\(r, t, ([-0-9.e]+)f\);", body)]
    return p, [*reversed(rest), top]          # c0 .. c7


def fma32(a, b, c):
    """fp32 fused multiply-add: the float32 product is exact in float64."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def poly32(z, p, coef):
    z = z.astype(np.float32)
    t = (np.float32(1) / fma32(np.float32(p), z, np.float32(1))).astype(np.float32)
    r = np.full_like(z, np.float32(coef[-1]))
    for c in reversed(coef[:-1]):
        r = fma32(r, t, np.full_like(z, np.float32(c)))
    return r.astype(np.float64)


def test_kernel_constants_are_float32_values_of_a_degree_7_fit():
    p, coef = kernel_constants()
    assert len(coef) == 8
    assert all(np.float32(c) == c for c in coef) and np.float32(p) == p


def test_kernel_polynomial_meets_the_stated_accuracy():
    """R(z) = erfcx(z / sqrt 2) / 2, so Q(z) = exp(-z^2/2) R(z); the fp32
    polynomial must be within 2^-20 relative of R on [0, 14] (the header's
    2^-14 allowance leaves room for the exp2 factor's own rounding), and it
    must stay positive wherever the exp2 factor does not vanish."""
    p, coef = kernel_constants()
    z = np.concatenate([np.linspace(0, 2, 20001), np.linspace(2, 14, 60001)])
    R = 0.5 * erfcx(z / np.sqrt(2))
    rel = np.abs(poly32(z, p, coef) - R) / R
    assert rel.max() < 2.0 ** -20, np.log2(rel.max())
    assert (poly32(np.linspace(0, 40, 4001), p, coef) > 0).all()


def test_fit_at_the_kernels_p_reproduces_the_constants():
    spec = importlib.util.spec_from_file_location("gelu_fit", os.path.join(CSRC, "gelu_fit.py"))
    gf = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(gf)
    p, coef = kernel_constants()
    # the scan's grid point that rounds to the kernel's fp32 p
    grid = np.linspace(0.30, 0.42, 25)
    p64 = grid[np.argmin(np.abs(grid.astype(np.float32) - np.float32(p)))]
    assert np.float32(p64) == np.float32(p)
    z = np.concatenate([np.linspace(0, 2, 40001), np.linspace(2, 14, 120001)])
    fitted, err = gf.fit(p64, z, 0.5 * erfcx(z / np.sqrt(2)))
    assert err < 2.0 ** -21
    # identical up to the last fp32 bits (least squares in another BLAS order)
    ulp = np.spacing(np.abs(np.asarray(coef, np.float32))).astype(np.float64)
    assert np.all(np.abs(fitted - np.asarray(coef)) <= 4 * ulp + 1e-12), (fitted, coef)
