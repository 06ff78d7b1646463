"""Derivation of the GELU constants used by the MFMA decode kernel.

For a >= 0 the upper tail of the normal distribution is written
1 - Phi(a) = 0.5 * exp(-f(a)), f(a) = -log(2 (1 - Phi(a))), and f is fitted
on [0, 6] by a degree-4 polynomial (Chebyshev basis, iteratively reweighted
towards the largest GELU error).  The kernel evaluates
GELU(x) = x * Phi(x) with Phi(x) = 1 - q for x >= 0 and q for x < 0,
q = exp2(-(f(min(|x|, 6)) * log2(e)) - 1), from half the argument: with
x2 = x / 2 and a = min(|x2|, 3) the exponent is a polynomial in a whose
coefficients are those in |x| times 2^k, and GELU(x) = x2 + |x2| (1 - 2 q).
Run: python fit_gelu_tail.py  (prints those half-argument coefficients,
already multiplied by -log2(e) with the -1 folded into the constant, and the
error of the form evaluated in fp32 against the exact erf form; then the
error of the decode kernel's two ways of handing GELU to an MFMA: the fp32
form rounded to bf16, and the packed-fp16 evaluation of gelu_half_pk, the
input converted to fp16 rounding toward zero and every step one fp16
rounding).
"""
import numpy as np
from scipy.special import log_ndtr, ndtr

X, N = 6.0, 4
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
half = (coef * 2.0 ** np.arange(N + 1)).astype(np.float32)
x = np.linspace(-12, 12, 480001)
x2 = (x / 2).astype(np.float32)
a = np.minimum(np.abs(x2), np.float32(X / 2))
e = np.zeros_like(a)
for c in half[::-1]:
    e = (e * a + c).astype(np.float32)
q = np.exp2(e).astype(np.float32)
g = x2 + np.abs(x2) * (np.float32(1) - 2 * q)
err = np.abs(g.astype(np.float64) - x * ndtr(x))
print("half-argument coefficients (ascending):", ", ".join(f"{c:.9e}f" for c in half))
print(f"max |GELU error| = {err.max():.3e}, max error/|x| = {np.max(err[np.abs(x) > 1e-3] / np.abs(x[np.abs(x) > 1e-3])):.3e}")


def bf16_rne(v):
    u = np.asarray(v, np.float32).view(np.uint32).astype(np.uint64)
    return (((u + 0x7FFF + ((u >> 16) & 1)) >> 16) << 16).astype(np.uint32).view(np.float32)


def f16(v):
    return np.asarray(v, np.float64).astype(np.float16)


def f16_rtz(v):
    v = np.asarray(v, np.float64)
    r = v.astype(np.float16)
    over = np.abs(r.astype(np.float64)) > np.abs(v)
    return np.where(over, np.nextafter(r, np.float16(0)), r).astype(np.float16)


exact = x * ndtr(x)
h = f16_rtz(x2)
ah = np.abs(h.astype(np.float64))
a16 = f16(np.minimum(ah, 3.0)).astype(np.float64)
e16 = np.zeros_like(a16)
for c in f16(half)[::-1]:
    e16 = f16(e16 * a16 + np.float64(c)).astype(np.float64)
q16 = f16(np.exp2(e16)).astype(np.float64)
g16 = f16(ah * f16(1.0 - 2.0 * q16).astype(np.float64) + h.astype(np.float64)).astype(np.float64)
m = np.abs(x) > 1e-3
for name, gv in (("fp32 form rounded to bf16", bf16_rne(g).astype(np.float64)), ("packed fp16 (gelu_half_pk)", g16)):
    r = (gv - exact)[m] / np.abs(x[m])
    print(f"{name}: max error/|x| = {np.abs(r).max():.3e}, rms = {np.sqrt(np.mean(r * r)):.3e}, mean = {r.mean():.2e}")
