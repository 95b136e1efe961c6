"""Coefficients of the erfc approximation used by gelu_erf (device_common.hpp).

erfc(x) for x = |z|/sqrt(2) is written t * 2^(Q(t) - z^2 log2(e)/2) with
t = 1 / (1 + |z| / (2 sqrt 2)); Q(t) = log2(erfcx(x) / t) is smooth on
t in [1/(1 + 14/(2 sqrt 2)), 1], and a degree-5 polynomial fitted there by
iteratively reweighted Chebyshev least squares (close to minimax) keeps the
fractional error of erfc below 8e-6 for |z| <= 14 (degree 7: 7e-7; the GELU
output is rounded to bf16, whose relative half-ulp is 2e-3).  Run: python
gelu_fit.py (needs numpy and scipy); prints the coefficients c0..c5 of Q and
the error.
"""
import numpy as np
import numpy.polynomial.chebyshev as C
from scipy.special import erfcx

P = 1.0 / (2.0 * np.sqrt(2.0))
DEG = 5


def fit(zmax=14.0, n=400001, iters=40):
    z = np.linspace(0.0, zmax, n)
    t = 1.0 / (1.0 + P * z)
    g = np.log2(erfcx(z / np.sqrt(2.0)) / t)
    tmin = t.min()
    u = (2 * t - (1 + tmin)) / (1 - tmin)
    w = np.ones_like(u)
    for _ in range(iters):
        c = C.chebfit(u, g, DEG, w=w)
        err = C.chebval(u, c) - g
        w = w * (1 + 4 * np.abs(err) / np.abs(err).max())
    a, b = 2 / (1 - tmin), -(1 + tmin) / (1 - tmin)
    coef = np.polynomial.Polynomial(C.cheb2poly(c))(np.polynomial.Polynomial([b, a])).coef
    rel = np.abs(np.polyval(coef[::-1], t) - g).max() * np.log(2.0)
    return coef, rel


if __name__ == "__main__":
    coef, rel = fit()
    for k, v in enumerate(coef):
        print(f"c{k} = {np.float32(v)!r}  # {v:.17g}")
    print(f"max fractional error of erfc: {rel:.2e}")
