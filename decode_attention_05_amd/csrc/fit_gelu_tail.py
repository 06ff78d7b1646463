"""Derivation of the GELU constants used by the MFMA decode kernel.

For a >= 0 the upper tail of the normal distribution is written
1 - Phi(a) = 0.5 * exp(-f(a)), f(a) = -log(2 (1 - Phi(a))), and f is fitted
on [0, 6] by a degree-6 polynomial (Chebyshev basis, iteratively reweighted
towards the largest GELU error).  The kernel evaluates
GELU(x) = x * Phi(x) with Phi(x) = 1 - q for x >= 0 and q for x < 0,
q = exp2(-(f(min(|x|, 6)) * log2(e)) - 1).
Run: python fit_gelu_tail.py  (prints the coefficients already multiplied by
-log2(e), with the -1 folded into the constant, and the measured error).
"""
import numpy as np
from scipy.special import log_ndtr, ndtr

X, N = 6.0, 6
xs = np.linspace(0, X, 60000)
f = -(np.log(2.0) + log_ndtr(-xs))
w = np.ones_like(xs)
for _ in range(80):
    cheb = np.polynomial.chebyshev.Chebyshev.fit(xs, f, N, domain=[0, X], w=w)
    e = np.abs(0.5 * np.exp(-cheb(xs)) - 0.5 * np.exp(-f)) * xs
    w *= 1 + 2 * e / e.max()
    w /= w.mean()
poly = cheb.convert(kind=np.polynomial.Polynomial, domain=[0, X], window=[0, X])
k = -1.0 / np.log(2.0)
coef = poly.coef * k
coef[0] -= 1.0
x = np.linspace(-12, 12, 480001)
a = np.minimum(np.abs(x), X)
q = np.exp2(np.polyval(coef[::-1], a))
g = x * np.where(x >= 0, 1 - q, q)
err = np.abs(g - x * ndtr(x))
print("coefficients (ascending):", ", ".join(f"{c:.9e}f" for c in coef))
print(f"max |GELU error| = {err.max():.3e}, max error/|x| = {np.max(err[np.abs(x) > 1e-3] / np.abs(x[np.abs(x) > 1e-3])):.3e}")
