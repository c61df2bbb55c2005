"""Fits the polynomial Q of the exact-GeLU kernels' erfc evaluation.

For x = k |z| with the fusions article's k = 0.70710678 and t = 1 / (1 + x/2):

    0.5 erfc(k |z|) = t * Q(t) * exp(-z^2 / 2)

so Q(t) = 0.5 erfc(x) exp(z^2 / 2) / t with z^2 = x^2 / k^2. Q is smooth and
bounded away from zero on t in [1/8, 1] (x <= 14; beyond, exp(-z^2/2) is
below 2^-190 and the kernels' product is zero), so a polynomial fitted for
relative error gives erfc to the same relative error everywhere, tails
included, and the factor exp(-z^2/2) is the one the derivative's Gaussian
term needs anyway.

Least squares with relative weights on Chebyshev points, degree 8 (kErfQ, for
fp32 outputs and every backward) and degree 5 (kErfQ5, for the forward with
bf16/fp16 outputs, where 3.5e-5 relative is far inside half an output ulp and
a product z Phi(z) has no cancellation to amplify it); prints the fp32
coefficients (lowest degree first) and the maximum relative error of the fp32
Horner evaluation on a dense grid. Needs numpy and scipy.

    python fit_erfc.py
"""
import numpy as np
from scipy.special import erfcx

K = 0.70710678
DEGREE = 8
DEGREE_HALF = 5
TMIN = 1.0 / 8.0


def target(t):
    x = 2.0 * (1.0 / t - 1.0)
    # 0.5 erfc(x) exp(x^2 / (2 k^2)) / t = 0.5 erfcx(x) exp(x^2 (1/(2k^2) - 1)) / t
    return 0.5 * erfcx(x) * np.exp(x * x * (0.5 / (K * K) - 1.0)) / t


def fit(degree=None):
    degree = DEGREE if degree is None else degree
    n = 6000
    j = np.arange(n)
    t = 0.5 * (1 + TMIN) + 0.5 * (1 - TMIN) * np.cos(np.pi * (j + 0.5) / n)
    q = target(t)
    V = np.vander(t, degree + 1, increasing=True) / q[:, None]
    c, *_ = np.linalg.lstsq(V, np.ones_like(t), rcond=None)
    return c.astype(np.float32)


def horner32(c32, t):
    t32 = t.astype(np.float32)
    p = np.full_like(t32, c32[-1])
    for ck in c32[-2::-1]:
        p = (p.astype(np.float64) * t32 + np.float64(ck)).astype(np.float32)  # one fma: exact product, one rounding
    return p.astype(np.float64)


if __name__ == "__main__":
    dense = np.linspace(TMIN, 1.0, 400001)
    for name, degree in (("kErfQ", DEGREE), ("kErfQ5", DEGREE_HALF)):
        c32 = fit(degree)
        rel = np.abs(horner32(c32, dense) / target(dense) - 1.0)
        print(f"{name}, degree {degree}, coefficients (t^0 first):")
        for ck in c32:
            print(f"  {float(ck):.9e}f  ({np.float32(ck).view(np.uint32):#010x})")
        print(f"max relative error of the fp32 evaluation on t in [{TMIN}, 1]: {rel.max():.3e}")
