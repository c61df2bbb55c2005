"""Pins for oracle32 (oracle/oracle32.c), the binary32 evaluation of the
oracle's formulas: a secondary statistic and the fp32 CPU baseline, never the
parity reference.

- Forward activations against torch float32 compositions of the formulas the
  Megatron-LM fusions walkthrough prints (section 4.2), which differ only in
  the library's tanh / erf / exp;
- dropout-add and squared ReLU: the same float operations done by numpy
  float32 (mask bits from the fp64 oracle's Philox), bit for bit, and float
  gradient sums equal to numpy's sequential float32 accumulation;
- everything against the fp64 oracle within the error bound of the float
  evaluation, so a dropped term or a wrong sign fails;
- the literal tanh derivative cancels in float in the negative tail (the
  reason the fp64 oracle, not oracle32, is the parity reference).
"""
import numpy as np
import pytest
import torch

import oracle
from oracle import oracle32

U = 2.0**-24
K, C, KD = 0.79788456, 0.044715, 0.1070322243


def rng(k):
    return np.random.default_rng(9300 + k)


def bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_val(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


def ulp_bf16(v):
    """Spacing of bf16 values at |v| (normal range)."""
    e = np.floor(np.log2(np.maximum(np.abs(v), 2.0**-126)))
    return 2.0 ** (e - 7)


def test_gelu_forward_is_the_printed_formula_in_float():
    x = (rng(1).standard_normal(20000) * 3).astype(np.float32)[None, :]
    t = torch.from_numpy(x)
    want_tanh = (t * 0.5 * (1.0 + torch.tanh(0.79788456 * t * (1 + 0.044715 * t * t)))).numpy()
    want_erf = (t * 0.5 * (1.0 + torch.erf(t * 0.70710678))).numpy()
    for exact, want in ((False, want_tanh), (True, want_erf)):
        got = oracle32.bias_gelu_fwd("f32", x, None, exact=exact)
        # the float operations are the same; only the library's tanh / erf differ (a few ulps of 1 + t)
        assert np.all(np.abs(got - want) <= 4 * U * np.abs(x) + 4 * np.spacing(np.abs(want))), exact


@pytest.mark.parametrize("exact", [False, True])
@pytest.mark.parametrize("dt", ["f32", "bf16"])
def test_gelu_within_float_bounds_of_the_fp64_oracle(dt, exact):
    r = rng(2)
    T, H = 64, 96
    yf = (r.standard_normal((T, H)) * 2).astype(np.float32).clip(-4, 4)
    gf = r.standard_normal((T, H)).astype(np.float32)
    bf = (r.standard_normal(H) * 0.1).astype(np.float32)
    enc = (lambda a: a) if dt == "f32" else bf16_bits
    dec = (lambda a: a.astype(np.float64)) if dt == "f32" else bf16_val
    y, g, b = enc(yf), enc(gf), enc(bf)
    z = dec(y) + dec(b)[None, :]
    out32 = oracle32.bias_gelu_fwd(dt, y, b, exact=exact)
    _, out64 = oracle.bias_gelu_fwd(dt, y, b, exact=exact)
    dg32, db32 = oracle32.bias_gelu_bwd(dt, g, y, b, exact=exact)
    _, d64, _, db64 = oracle.bias_gelu_bwd(dt, g, y, b, exact=exact)
    store = (lambda v: 0.0) if dt == "f32" else ulp_bf16
    # forward: x * 0.5 * (1 + t) with t off by a few ulps and each product rounded
    e_fwd = 16 * U * np.abs(z) + store(out64)
    assert np.all(np.abs(dec(out32) - out64) <= e_fwd)
    # backward: |g| times the size of the derivative's terms, each a few roundings off
    if exact:
        scale = 0.5 * (1 + np.abs(np.tanh(z))) + np.abs(z) * 0.3989423 * np.exp(-0.5 * z * z)
    else:
        scale = 1 + 0.5 * np.abs(z) * (K + KD * z * z)
    e_bwd = 32 * U * np.abs(dec(g)) * scale
    assert np.all(np.abs(dec(dg32) - d64) <= e_bwd + store(d64))
    assert np.all(np.abs(db32 - db64) <= T * U * np.sum(np.abs(d64), 0) + np.sum(e_bwd, 0))


def test_literal_tanh_derivative_cancels_in_the_float_tail():
    """Once tanhf(u) rounds to -1, 0.5 (1 + t) and 1 - t^2 are exactly 0 in
    float, so the literal derivative is 0 where the true one is not."""
    z = np.linspace(-12.0, -9.5, 64).astype(np.float32)[None, :]
    g = np.ones_like(z)
    dg32, _ = oracle32.bias_gelu_bwd("f32", g, z, None)
    _, d64, _, _ = oracle.bias_gelu_bwd("f32", g, z, None)
    assert np.all(dg32 == 0.0) and np.all(d64 != 0.0)
    # in the ordinary range the two agree to float accuracy
    z = np.linspace(-3.0, 3.0, 601).astype(np.float32)[None, :]
    dg32, _ = oracle32.bias_gelu_bwd("f32", np.ones_like(z), z, None)
    _, d64, _, _ = oracle.bias_gelu_bwd("f32", np.ones_like(z), z, None)
    assert np.max(np.abs(dg32 - d64)) < 1e-6


@pytest.mark.parametrize("rdt", ["bf16", "f32"])
def test_dropout_add_is_float_arithmetic_bit_for_bit(rdt):
    r = rng(3)
    T, H, p, seed, off = 48, 72, 0.3, 1234, 5
    xf = (r.standard_normal((T, H)) * 2).astype(np.float32)
    bf = (r.standard_normal(H) * 0.3).astype(np.float32)
    rf = r.standard_normal((T, H)).astype(np.float32)
    gf = r.standard_normal((T, H)).astype(np.float32)
    x, b, g = bf16_bits(xf), bf16_bits(bf), bf16_bits(gf)
    res = bf16_bits(rf) if rdt == "bf16" else rf
    keep = np.unpackbits(oracle.dropout_mask(T, H, p, seed, off), bitorder="little")[:T * H].reshape(T, H) == 1
    s = np.float32(oracle.keep_scale(p))
    xv, bv, gv = (bf16_val(a).astype(np.float32) for a in (x, b, g))
    rv = bf16_val(res).astype(np.float32) if rdt == "bf16" else bf16_val(bf16_bits(rf)).astype(np.float32)
    z = xv + bv[None, :]
    want = bf16_bits(rv + np.where(keep, z * s, np.float32(0)))
    got = oracle32.bias_dropout_add("bf16", x, b, res, rdt, True, p, seed, off)
    assert np.array_equal(got, want)
    assert np.array_equal(oracle32.bias_dropout_add("bf16", x, b, res, rdt, False), bf16_bits(rv + z))
    dx, dres, db = oracle32.bias_dropout_add_bwd("bf16", g, rdt, p, seed, off)
    v = np.where(keep, gv * s, np.float32(0))
    assert np.array_equal(dx, bf16_bits(v))
    assert np.array_equal(dres, g if rdt == "bf16" else gv)
    assert np.array_equal(db, np.add.accumulate(v, axis=0, dtype=np.float32)[-1])
    # the fp64 oracle's dx agrees wherever the float product rounds to the same bf16
    dx64, _, _, _ = oracle.bias_dropout_add_bwd("bf16", g, rdt, p, seed, off)
    assert np.all(np.abs(bf16_val(dx) - bf16_val(dx64)) <= ulp_bf16(bf16_val(dx64)))


def test_squared_relu_is_float_arithmetic_bit_for_bit():
    r = rng(4)
    T, H = 40, 64
    x, g = bf16_bits(r.standard_normal((T, H)) * 2), bf16_bits(r.standard_normal((T, H)))
    w = r.random(T).astype(np.float32)
    xv, gv = bf16_val(x).astype(np.float32), bf16_val(g).astype(np.float32)
    rl = np.maximum(xv, np.float32(0))
    assert np.array_equal(oracle32.weighted_squared_relu_fwd("bf16", x, w, "f32"), bf16_bits(rl * rl * w[:, None]))
    dx, dw = oracle32.weighted_squared_relu_bwd("bf16", g, x, w, "f32")
    assert np.array_equal(dx, bf16_bits(gv * w[:, None] * np.float32(2) * rl))
    assert np.array_equal(dw, np.add.accumulate(gv * rl * rl, axis=1, dtype=np.float32)[:, -1])


@pytest.mark.parametrize("act", ["swiglu", "geglu"])
def test_glu_within_float_bounds_of_the_fp64_oracle(act):
    r = rng(5)
    T, H = 32, 80
    inp = bf16_bits((r.standard_normal((T, 2 * H)) * 2).clip(-4, 4))
    b = bf16_bits(r.standard_normal(2 * H) * 0.1)
    g = bf16_bits(r.standard_normal((T, H)))
    w = bf16_bits(r.random(T)) if act == "swiglu" else None
    out32 = oracle32.bias_glu_fwd(act, "bf16", inp, b, w)
    _, o64 = oracle.bias_glu_fwd(act, "bf16", inp, b, w)
    assert np.all(np.abs(bf16_val(out32) - o64) <= 16 * U * np.abs(o64) + 1e-30 + ulp_bf16(o64))
    din32, db32, dw32 = oracle32.bias_glu_bwd(act, "bf16", g, inp, b, w)
    _, d64, mag, db64, dw64 = oracle.bias_glu_bwd(act, "bf16", g, inp, b, w)
    e = 64 * U * mag
    assert np.all(np.abs(bf16_val(din32) - d64) <= e + ulp_bf16(d64))
    assert np.all(np.abs(db32 - db64) <= T * U * np.sum(np.abs(d64), 0) + np.sum(e, 0))
    if act == "swiglu":
        assert np.all(np.abs(dw32 - dw64) <= 2 * H * U * np.sum(np.abs(d64), 1) + 1e-6)
    # forward in float, against torch float32 (silu from the library)
    a = torch.from_numpy(bf16_val(inp)[:, :H] + bf16_val(b)[None, :H]).float()
    bb = torch.from_numpy(bf16_val(inp)[:, H:] + bf16_val(b)[None, H:]).float()
    if act == "swiglu":
        ref = torch.nn.functional.silu(a) * bb * torch.from_numpy(bf16_val(w)).float()[:, None]
    else:
        ref = a * 0.5 * (1.0 + torch.tanh(0.79788456 * a * (1 + 0.044715 * a * a))) * bb
    assert np.all(np.abs(bf16_val(out32) - ref.double().numpy()) <= 8 * U * np.abs(ref.double().numpy())
                  + ulp_bf16(ref.double().numpy()))


@pytest.mark.parametrize("dt,rdt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")])
def test_layer_norm_within_float_bounds_of_the_fp64_oracle(dt, rdt):
    r = rng(6)
    T, H = 24, 520
    enc = {"bf16": bf16_bits, "f32": lambda a: np.asarray(a, np.float32)}
    dec = {"bf16": bf16_val, "f32": lambda a: a.astype(np.float64)}
    x, res = enc[dt](r.standard_normal((T, H)) + 0.5), enc[rdt](r.standard_normal((T, H)))
    gm, bt = enc[dt](1 + 0.2 * r.standard_normal(H)), enc[dt](0.1 * r.standard_normal(H))
    h32, y32, mean32, rstd32 = oracle32.add_layer_norm_fwd(dt, x, res, rdt, gm, bt)
    h64, y64o, y64, mag, mean64, rstd64 = oracle.add_layer_norm_fwd(dt, x, res, rdt, gm, bt)
    assert np.array_equal(h32, h64)  # one rounding of an exact float sum
    store = (lambda v: 0.0) if dt == "f32" else ulp_bf16
    Kb = 4 * H  # sequential float row sums: depth H
    assert np.all(np.abs(dec[dt](y32) - y64) <= Kb * U * mag + store(y64))
    assert np.all(np.abs(mean32 - mean64) <= Kb * U * np.mean(np.abs(dec[dt](h64)), 1))
    assert np.all(np.abs(rstd32 - rstd64) <= Kb * U * rstd64)
    dy, up = enc[dt](r.standard_normal((T, H))), enc[rdt](0.5 * r.standard_normal((T, H)))
    dx32, dres32, dg32, db32 = oracle32.add_layer_norm_bwd(dt, dy, h64, gm, dh_in=up, res_dt=rdt)
    _, dx64, bmag, _, dg64, db64 = oracle.add_layer_norm_bwd(dt, dy, h64, gm, dh_in=up, res_dt=rdt)
    assert np.all(np.abs(dec[dt](dx32) - dx64) <= Kb * U * bmag + store(dx64))
    assert np.all(np.abs(dec[rdt](dres32) - dx64) <= Kb * U * bmag + (store(dx64) if rdt == "bf16" else 0.0))
    dyv = dec[dt](dy)
    assert np.all(np.abs(db32 - db64) <= T * U * np.sum(np.abs(dyv), 0) + 1e-30)
    assert np.all(np.abs(dg32 - dg64) <= (T + Kb) * U * np.sum(np.abs(dyv) * (np.abs(dec[dt](h64)) + 1)
                                                                * rstd64[:, None], 0))


def test_oracle32_refuses_what_it_does_not_evaluate():
    with pytest.raises(ValueError):
        oracle32.bias_gelu_fwd("f64", np.zeros((1, 4)), None)
    with pytest.raises(ValueError):
        oracle32.bias_dropout_add_bwd("bf16", np.zeros((1, 8), np.uint16), "bf16", 1.5, 0)
