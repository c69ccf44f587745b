"""Coefficients of the erfc approximation used by the GELU epilogue.

Form: for z >= 0, t = 1 / (1 + z/2) and erfc(z) ~= t * exp(-z^2 + P(t)), the
form of the "erfcc" routine of Numerical Recipes (2nd ed., section 6.2), with
our own polynomial: P of degree 5 fitted to g(t) = ln(erfc(z) / t) + z^2 on
z in [0, 10] (t in [1/6, 1]; beyond z = 10, erfc(z) < 3e-45 and the fp32
result is zero either way) by Lawson's iteratively reweighted least squares
toward the minimax fit, in the Chebyshev basis, then converted to powers of
t for Horner evaluation.  The relative error of erfc is exp(P - g) - 1, so
max |P - g| bounds it.  The kernel evaluates erfc(z)/2 as t * 2^(-log2(e) z^2
+ Q(t)) with Q = log2(e) P - 1 (base-2 exponential, the halving in the
constant term), so it takes Q's coefficients, printed last.

    python gelu_fit.py        # prints the coefficients (highest power first)
"""
import numpy as np
from scipy.special import erfc

DEGREE = 5
Z_MAX = 10.0


def fit(degree: int = DEGREE, n: int = 200001, iters: int = 60):
    z = np.linspace(0.0, Z_MAX, n)
    t = 1.0 / (1.0 + z / 2.0)
    g = np.log(erfc(z) / t) + z * z
    lo, hi = 1.0 / (1.0 + Z_MAX / 2.0), 1.0
    x = (2.0 * t - (lo + hi)) / (hi - lo)
    w = np.ones_like(t)
    for _ in range(iters):
        c = np.polynomial.chebyshev.chebfit(x, g, degree, w=np.sqrt(w))
        e = np.polynomial.chebyshev.chebval(x, c) - g
        w = w * np.abs(e)
        w /= w.sum()
    # Chebyshev series in x -> power series in t
    cheb = np.polynomial.Chebyshev(c, domain=[lo, hi])
    power = cheb.convert(kind=np.polynomial.Polynomial).coef   # a_0 .. a_d in powers of t
    return power, float(np.abs(e).max())


def horner_f32(coef_high_first, t):
    p = np.float32(coef_high_first[0])
    for a in coef_high_first[1:]:
        p = np.float32(np.float32(p * t) + np.float32(a))
    return p


if __name__ == "__main__":
    power, err = fit()
    high_first = power[::-1]
    print("max |P - g| (fp64):", f"{err:.3e}")
    print("coefficients, highest power first:")
    for a in high_first:
        print(f"  {np.float32(a)!r}")
    z = np.linspace(0.0, Z_MAX, 20001)
    t = (1.0 / (1.0 + z / 2.0)).astype(np.float32)
    g = np.log(erfc(z) / t.astype(np.float64)) + z * z
    p32 = np.array([horner_f32(high_first.astype(np.float32), tt) for tt in t], dtype=np.float64)
    print("max |P_fp32 - g|:", f"{np.abs(p32 - g).max():.3e}")
    q = high_first / np.log(2.0)
    q[-1] -= 1.0
    print("coefficients of Q = log2(e) P - 1, highest power first:")
    for a in q:
        print(f"  {np.float32(a)!r}")
