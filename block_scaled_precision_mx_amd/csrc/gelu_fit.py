"""Derivation of the fp32 GELU used by the fused fc1 epilogue (gemm_mx.hip,
gelu_f32): prints its constants and their accuracy. Not used at run time.

GELU(h) = h Phi(h). With z = |h| and Q(z) = Phi(-z) (the normal upper tail),
Phi(h) = 1 - Q(z) for h >= 0 and Q(z) for h < 0. Q(z) = exp(-z^2/2) R(z),
where R(z) = erfcx(z / sqrt 2) / 2 is smooth and decreases from 1/2 like
1 / (z sqrt(2 pi)). R is fitted as a polynomial of degree 7 in
t = 1 / (1 + p z) by weighted least squares for relative error, with
Lawson's reweighting towards the minimax solution, on z in [0, 14] (beyond
14, |GELU| < 2^-140); p is scanned. The kernel evaluates the polynomial in
fp32 by Horner with fused multiply-adds.
"""
import numpy as np
from scipy.special import erfcx

DEG = 7


def fit(p: float, z: np.ndarray, R: np.ndarray):
    t = 1.0 / (1.0 + p * z)
    V = np.vander(t, DEG + 1, increasing=True)
    w = 1.0 / R
    for _ in range(60):
        coef, *_ = np.linalg.lstsq(V * w[:, None], R * w, rcond=None)
        err = (V @ coef - R) / R
        w = w * (1 + 50 * np.abs(err) / np.abs(err).max())
    return coef, np.abs(err).max()


def main():
    z = np.concatenate([np.linspace(0, 2, 40001), np.linspace(2, 14, 120001)])
    R = 0.5 * erfcx(z / np.sqrt(2))
    best = min((fit(p, z, R) + (p,) for p in np.linspace(0.30, 0.42, 25)), key=lambda r: r[1])
    coef, err, p = best
    c32, p32, z32 = coef.astype(np.float32), np.float32(p), z.astype(np.float32)
    t = (np.float32(1) / (np.float32(1) + p32 * z32)).astype(np.float32)
    acc = np.full_like(t, c32[-1])
    for k in range(DEG - 1, -1, -1):
        acc = (acc.astype(np.float64) * t + np.float64(c32[k])).astype(np.float32)   # fma, one rounding
    rel32 = np.abs((acc - R) / R).max()
    print(f"p = {float(p32)!r}  fit error 2^{np.log2(err):.1f}, fp32 evaluation 2^{np.log2(rel32):.1f}")
    for k, v in enumerate(c32):
        print(f"c{k} = {float(v)!r}")


if __name__ == "__main__":
    main()
