"""Two-sided pins of the oracle's cancellation scales ("mag"), which widen the
parity floor where an fp32 evaluation cancels. An over-estimated mag would
silently loosen every floor pass, so each one is pinned from above as well as
from below, against quantities the oracle's code does not produce:

* where no cancellation can occur (all summands of the derivative share a
  sign), mag is the larger of two same-signed summands, so
  |d|/2 <= mag <= |d| with d the gradient, itself pinned by finite
  differences in test_oracle_ops.py;
* everywhere, mag equals the larger summand of the derivative as printed
  (Megatron-LM fusions walkthrough, section 4.2; SiLU's derivative
  sigma (1 + a (1 - sigma))), evaluated here in 50-digit arithmetic (mpmath)
  from the literal formulas, on |z| <= 8;
* dropout-add: mag is the largest of |r'|, |z s|, |x s|, |b s| for a kept
  element and |r'| for a dropped one, checked against numpy.
"""
import mpmath as mp
import numpy as np

import oracle

K, C, KD = 0.79788456, 0.044715, 0.1070322243  # printed constants (walkthrough section 4.2)


def rng(k):
    return np.random.default_rng(9100 + k)


mp.mp.dps = 50


def _each(f, z):
    """f(mpf) -> (s1, s2) applied elementwise, back to float64 arrays."""
    out = [f(mp.mpf(float(v))) for v in np.asarray(z).reshape(-1)]
    s1 = np.array([float(a) for a, _ in out]).reshape(np.shape(z))
    s2 = np.array([float(b) for _, b in out]).reshape(np.shape(z))
    return s1, s2


def gelu_summands(z):
    def f(v):
        u = K * v * (1 + C * v * v)
        t = mp.tanh(u)
        return abs(mp.mpf("0.5") * (1 + t)), abs(mp.mpf("0.5") * v * (1 - t * t) * (K + KD * v * v))
    return _each(f, z)


def erf_summands(z):
    def f(v):
        return (abs(mp.mpf("0.5") * (1 + mp.erf(mp.mpf("0.70710678") * v))),
                abs(v * mp.mpf("0.3989423") * mp.exp(-v * v / 2)))
    return _each(f, z)


def silu_summands(a):
    def f(v):
        s = 1 / (1 + mp.exp(-v))
        return s, abs(s * v * (1 - s))
    return _each(f, a)


def test_gelu_bwd_mag_two_sided():
    r = rng(1)
    y = np.concatenate([np.linspace(-8, 8, 1601), r.standard_normal(800) * 2]).clip(-8, 8)[None, :]
    g = r.standard_normal(y.shape)
    for exact, summ in ((False, gelu_summands), (True, erf_summands)):
        _, d64, mag, _ = oracle.bias_gelu_bwd("f64", g, y, None, exact=exact)
        s1, s2 = summ(y)
        want = np.abs(g) * np.maximum(s1, s2)
        assert np.allclose(mag, want, rtol=1e-9, atol=1e-300), exact
        pos = y >= 0  # both summands >= 0: no cancellation
        assert np.all(mag[pos] <= np.abs(d64[pos]) * (1 + 1e-12))
        assert np.all(mag[pos] >= np.abs(d64[pos]) / 2 * (1 - 1e-12))


def test_glu_bwd_mag_two_sided():
    r = rng(2)
    T, H = 8, 128
    a = np.concatenate([np.linspace(-8, 8, T * H // 2), r.standard_normal(T * H // 2) * 2]).clip(-8, 8)
    b = r.standard_normal(T * H)
    x = np.concatenate([a.reshape(T, H), b.reshape(T, H)], axis=1)
    g = r.standard_normal((T, H))
    w = r.random(T)
    for act, summ in (("swiglu", silu_summands), ("geglu", gelu_summands)):
        _, d64, mag, _, _ = oracle.bias_glu_bwd(act, "f64", g, x, None, w if act == "swiglu" else None, "f64")
        wt = w[:, None] if act == "swiglu" else 1.0
        s1, s2 = summ(x[:, :H])
        want_a = np.abs(g * wt * x[:, H:]) * np.maximum(s1, s2)
        assert np.allclose(mag[:, :H], want_a, rtol=1e-9, atol=1e-300), act
        # the up half has no cancellation: its scale is its own magnitude
        assert np.allclose(mag[:, H:], np.abs(d64[:, H:]), rtol=1e-12, atol=0), act
        pos = x[:, :H] >= 0
        da = np.abs(d64[:, :H])
        assert np.all(mag[:, :H][pos] <= da[pos] * (1 + 1e-12)), act
        assert np.all(mag[:, :H][pos] >= da[pos] / 2 * (1 - 1e-12)), act


def test_bda_mag_two_sided():
    r = rng(3)
    T, H = 64, 128
    x = r.standard_normal((T, H)) * 3
    b = r.standard_normal(H) * 0.5
    res = r.standard_normal((T, H))
    p, seed = 0.3, 77
    out, out64, mag = oracle.bias_dropout_add("f64", x, b, res, "f64", True, p, seed, 0)
    s = float(oracle.keep_scale(p))
    bits = oracle.dropout_mask(T, H, p, seed, 0)
    keep = np.unpackbits(bits, bitorder="little")[:T * H].reshape(T, H).astype(bool)
    z = x + b
    kept_m = np.maximum.reduce([np.abs(res), np.abs(z * s), np.abs(x * s), np.abs(np.broadcast_to(b, (T, H)) * s)])
    want = np.where(keep, kept_m, np.abs(res))
    assert np.array_equal(mag, want)
    # where r' and z s share a sign nothing cancels: mag <= |out| <= 2 mag (plus the x, b split)
    same = keep & (np.sign(res) == np.sign(z)) & (np.sign(x) == np.sign(b))
    assert np.all(mag[same] <= np.abs(out64[same]) * (1 + 1e-12))
