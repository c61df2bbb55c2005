"""Pins for the oracle's fused ops (bias broadcast, dropout-add, gated units, gradients).

- forward ops against torch float64 CPU compositions of library routines
  (F.gelu / F.silu / torch.chunk with broadcasting), which fixes the bias
  broadcast and the gate/up half order;
- backward ops against a brute-force finite-difference Jacobian of the
  oracle's own forward op (double storage), contracted with g, over every
  input, bias and weight element of small tensors;
- reductions (dbias, dweights) against brute-force column / row sums;
- dropout-add: p = 0 equals inference bit for bit, p = 1 leaves the cast
  residual, every element agrees with its mask bit, the residual cast equals
  torch's, and row sampling (row0) reproduces the full evaluation;
- special cases: b = 1 reduces SwiGLU to silu and GEGLU to the tanh GeLU;
  weights = 1 reduce weighted SwiGLU to the unweighted one; weighted =
  unweighted times weights, forward and gradients.
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rng(seed):
    return np.random.default_rng(seed)


def bf16_bits(a_f32: np.ndarray) -> np.ndarray:
    return torch.from_numpy(np.ascontiguousarray(a_f32, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()


# ---------------------------------------------------------------- GeLU

def test_gelu_fwd_matches_torch_broadcast():
    r = rng(1)
    y = r.standard_normal((64, 136)).astype(np.float32) * 3
    b = (r.standard_normal(136) * 0.5).astype(np.float32)
    out, out64 = oracle.bias_gelu_fwd("f32", y, b)
    ref = F.gelu(torch.from_numpy(y).double() + torch.from_numpy(b).double(), approximate="tanh").numpy()
    mask = np.abs(y + b) < 5  # where torch's literal double evaluation is accurate
    assert np.all(np.abs(out64 - ref)[mask] <= 3e-8 * np.abs(ref)[mask] + 1e-14)
    assert np.array_equal(out, out64.astype(np.float32))


def test_gelu_fwd_bias_none_is_zero_bias():
    r = rng(2)
    y = bf16_bits(r.standard_normal((8, 24)).astype(np.float32))
    a, _ = oracle.bias_gelu_fwd("bf16", y, None)
    b, _ = oracle.bias_gelu_fwd("bf16", y, np.zeros(24, np.uint16))
    assert np.array_equal(a, b)


def _fd_grad(f, x, h_rel=1e-6):
    """Central-difference gradient of the scalar function f at the float64 array x."""
    g = np.zeros_like(x)
    flat = x.reshape(-1)
    gf = g.reshape(-1)
    for k in range(flat.size):
        h = h_rel * max(1.0, abs(flat[k]))
        old = flat[k]
        flat[k] = old + h
        fp = f()
        flat[k] = old - h
        fm = f()
        flat[k] = old
        gf[k] = (fp - fm) / (2 * h)
    return g


def _close(an, fd, scale):
    # central differences in double with h ~ 1e-6: error ~1e-10 relative + 1e-10 abs
    return np.abs(an - fd) <= 1e-7 * np.abs(fd) + 1e-8 * scale


def test_gelu_bwd_brute_force_jacobian_4x8():
    r = rng(3)
    y = r.standard_normal((4, 8)) * 2
    b = r.standard_normal(8) * 0.3
    g = r.standard_normal((4, 8))
    _, d64, _, db64 = oracle.bias_gelu_bwd("f64", g, y, b)

    def loss():
        _, o = oracle.bias_gelu_fwd("f64", y, b)
        return float(np.sum(g * o))

    fy = _fd_grad(loss, y)
    fb = _fd_grad(loss, b)
    assert np.all(_close(d64, fy, 1.0))
    assert np.all(_close(db64, fb, 1.0))


def test_gelu_bwd_dbias_is_column_sum():
    r = rng(4)
    y = bf16_bits(r.standard_normal((33, 40)).astype(np.float32))
    g = bf16_bits(r.standard_normal((33, 40)).astype(np.float32))
    b = bf16_bits((r.standard_normal(40) * 0.02).astype(np.float32))
    dg, d64, mag, db = oracle.bias_gelu_bwd("bf16", g, y, b)
    assert np.allclose(db, d64.sum(axis=0), rtol=1e-13, atol=1e-13)
    assert np.all(mag >= np.abs(d64) / 2 - 1e-300)  # the larger summand bounds half the sum


def test_gelu_bwd_empty_tokens():
    y = np.zeros((0, 16), np.float32)
    _, _, _, db = oracle.bias_gelu_bwd("f32", y, y, np.zeros(16, np.float32))
    assert np.array_equal(db, np.zeros(16))


def test_gelu_nan_propagates():
    y = np.array([[np.nan, 1.0, -1.0, 0.0]], np.float32)
    out, _ = oracle.bias_gelu_fwd("f32", y, None)
    assert math.isnan(out[0, 0]) and not np.any(np.isnan(out[0, 1:]))


# ---------------------------------------------------------------- dropout-add

def _bda_inputs(seed, T=16, H=64, res_dt="f32"):
    r = rng(seed)
    x = bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    b = bf16_bits((r.standard_normal(H) * 0.02).astype(np.float32))
    res32 = r.standard_normal((T, H)).astype(np.float32)
    res = res32 if res_dt == "f32" else bf16_bits(res32)
    return x, b, res


@pytest.mark.parametrize("res_dt", ["f32", "bf16"])
def test_bda_p0_equals_inference_bitwise(res_dt):
    x, b, res = _bda_inputs(5, res_dt=res_dt)
    tr, _, _ = oracle.bias_dropout_add("bf16", x, b, res, res_dt, True, 0.0, 1234, 0)
    inf, _, _ = oracle.bias_dropout_add("bf16", x, b, res, res_dt, False)
    assert np.array_equal(tr, inf)


def test_bda_p1_leaves_cast_residual():
    x, b, res = _bda_inputs(6)
    out, _, _ = oracle.bias_dropout_add("bf16", x, b, res, "f32", True, 1.0, 1234, 0)
    cast = bf16_bits(res)  # torch's fp32 -> bf16 cast (round to nearest even)
    want = np.where(cast == 0x8000, np.uint16(0), cast)  # r' + 0 turns -0 into +0
    assert np.array_equal(out, want)


@pytest.mark.parametrize("p", [0.1, 0.5, 1 - 2.0**-24])
@pytest.mark.parametrize("offset", [0, 7, 2**33])
def test_bda_elements_follow_mask_bits(p, offset):
    T, H, seed = 16, 64, 1234
    x, b, res = _bda_inputs(7, T, H)
    out, out64, mag = oracle.bias_dropout_add("bf16", x, b, res, "f32", True, p, seed, offset)
    bits = np.unpackbits(oracle.dropout_mask(T, H, p, seed, offset), bitorder="little")[:T * H].reshape(T, H)
    rprime = bf16_value(bf16_bits(res))
    z = bf16_value(x) + bf16_value(b)[None, :]
    s = float(np.float32(1.0 / (1.0 - float(np.float32(p)))))
    want = np.where(bits == 1, rprime + z * s, rprime + 0.0)
    assert np.array_equal(out64, want)
    assert np.all(mag >= np.abs(rprime))


def test_bda_residual_same_dtype_is_not_recast():
    x, b, res = _bda_inputs(8, res_dt="bf16")
    out, out64, _ = oracle.bias_dropout_add("bf16", x, b, res, "bf16", False)
    assert np.array_equal(out64, bf16_value(res) + (bf16_value(x) + bf16_value(b)[None, :]))


def test_bda_fp32_inference_is_plain_sum():
    r = rng(9)
    x = r.standard_normal((8, 32)).astype(np.float32)
    b = r.standard_normal(32).astype(np.float32)
    res = r.standard_normal((8, 32)).astype(np.float32)
    out, out64, _ = oracle.bias_dropout_add("f32", x, b, res, "f32", False)
    assert np.array_equal(out64, res.astype(np.float64) + (x.astype(np.float64) + b.astype(np.float64)))
    assert np.array_equal(out, out64.astype(np.float32))


def test_bda_row_sampling_reproduces_full_evaluation():
    T, H = 24, 40
    x, b, res = _bda_inputs(10, T, H)
    full, _, _ = oracle.bias_dropout_add("bf16", x, b, res, "f32", True, 0.3, 99, 5)
    part, _, _ = oracle.bias_dropout_add("bf16", x[9:17], b, res[9:17], "f32", True, 0.3, 99, 5, row0=9)
    assert np.array_equal(full[9:17], part)
    mfull = np.unpackbits(oracle.dropout_mask(T, H, 0.3, 99, 5), bitorder="little")[:T * H]
    mpart = np.unpackbits(oracle.dropout_mask(8, H, 0.3, 99, 5, row0=9), bitorder="little")[:8 * H]
    assert np.array_equal(mfull[9 * H:17 * H], mpart)


def test_bda_dropped_nan_does_not_propagate():
    T, H, p, seed = 4, 64, 0.5, 3
    x, b, res = _bda_inputs(11, T, H)
    bits = np.unpackbits(oracle.dropout_mask(T, H, p, seed, 0), bitorder="little")[:T * H].reshape(T, H)
    x = x.copy()
    x[bits == 0] = 0x7FC0  # NaN wherever the element is dropped
    x[0, np.argmax(bits[0])] = 0x7FC0  # and one kept element
    out, _, _ = oracle.bias_dropout_add("bf16", x, b, res, "f32", True, p, seed, 0)
    vals = bf16_value(out)
    assert np.isnan(vals).sum() == 1


def test_bda_rejects_bad_probability():
    x, b, res = _bda_inputs(12, 2, 8)
    for p in (-0.1, 1.5, float("nan")):
        with pytest.raises(ValueError):
            oracle.bias_dropout_add("bf16", x, b, res, "f32", True, p, 1, 0)


# ---------------------------------------------------------------- gated units

@pytest.mark.parametrize("act", ["swiglu", "geglu"])
def test_glu_fwd_matches_torch_chunk_composition(act):
    r = rng(13)
    T, H = 12, 40
    x = r.standard_normal((T, 2 * H)).astype(np.float32) * 2
    b = (r.standard_normal(2 * H) * 0.1).astype(np.float32)
    out, out64 = oracle.bias_glu_fwd(act, "f32", x, b)
    y1, y2 = torch.chunk(torch.from_numpy(x).double() + torch.from_numpy(b).double(), 2, -1)
    ref = (F.silu(y1) if act == "swiglu" else F.gelu(y1, approximate="tanh")) * y2
    tol = 1e-14 if act == "swiglu" else 3e-8
    ok = np.abs(y1.numpy()) < 5  # where torch's literal tanh form is accurate
    assert np.all((np.abs(out64 - ref.numpy()) <= tol * np.abs(ref.numpy()) + 1e-14)[ok])


@pytest.mark.parametrize("act", ["swiglu", "geglu"])
def test_glu_with_unit_up_half_is_the_activation(act):
    r = rng(14)
    T, H = 8, 16
    a = r.standard_normal((T, H)) * 3
    x = np.concatenate([a, np.ones((T, H))], axis=1)
    _, out64 = oracle.bias_glu_fwd(act, "f64", x, None)
    at = torch.from_numpy(a)
    ref = (F.silu(at) if act == "swiglu" else F.gelu(at, approximate="tanh")).numpy()
    tol = 1e-15 if act == "swiglu" else 3e-8
    # torch's literal double evaluation of the tanh form cancels below z ~ -5
    ok = np.ones_like(a, bool) if act == "swiglu" else np.abs(a) < 5
    assert np.all((np.abs(out64 - ref) <= tol * np.abs(ref) + 1e-300)[ok])


def test_weighted_swiglu_equals_unweighted_times_weights():
    r = rng(15)
    T, H = 16, 24
    x = r.standard_normal((T, 2 * H))
    b = r.standard_normal(2 * H) * 0.02
    w = r.random(T)
    g = r.standard_normal((T, H))
    _, o_u = oracle.bias_glu_fwd("swiglu", "f64", x, b)
    _, o_w = oracle.bias_glu_fwd("swiglu", "f64", x, b, w)
    assert np.allclose(o_w, o_u * w[:, None], rtol=1e-15, atol=0)
    _, d_u, _, db_u, _ = oracle.bias_glu_bwd("swiglu", "f64", g, x, b)
    _, d_w, _, db_w, dw = oracle.bias_glu_bwd("swiglu", "f64", g, x, b, w)
    assert np.allclose(d_w, d_u * w[:, None], rtol=1e-14, atol=1e-300)
    # the weights gradient is the row sum of g times the unweighted output
    assert np.allclose(dw, np.sum(g * o_u, axis=1), rtol=1e-12, atol=1e-14)
    assert np.allclose(db_w, d_w.sum(axis=0), rtol=1e-12, atol=1e-14)


def test_unit_weights_reduce_to_unweighted_bitwise():
    r = rng(16)
    T, H = 8, 32
    x = bf16_bits(r.standard_normal((T, 2 * H)).astype(np.float32))
    g = bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    ones = np.full(T, 0x3F80, np.uint16)  # bf16 1.0
    a, _ = oracle.bias_glu_fwd("swiglu", "bf16", x, None)
    b, _ = oracle.bias_glu_fwd("swiglu", "bf16", x, None, ones)
    assert np.array_equal(a, b)
    da, *_ = oracle.bias_glu_bwd("swiglu", "bf16", g, x, None)
    db, *_ = oracle.bias_glu_bwd("swiglu", "bf16", g, x, None, ones)
    assert np.array_equal(da, db)


@pytest.mark.parametrize("act,weighted", [("swiglu", False), ("swiglu", True), ("geglu", False)])
def test_glu_bwd_brute_force_jacobian_4x16(act, weighted):
    r = rng(17)
    T, H = 4, 8
    x = r.standard_normal((T, 2 * H)) * 2
    b = r.standard_normal(2 * H) * 0.3
    w = r.random(T) + 0.1 if weighted else None
    g = r.standard_normal((T, H))
    _, din64, _, db64, dw64 = oracle.bias_glu_bwd(act, "f64", g, x, b, w)

    def loss():
        _, o = oracle.bias_glu_fwd(act, "f64", x, b, w)
        return float(np.sum(g * o))

    assert np.all(_close(din64, _fd_grad(loss, x), 1.0))
    assert np.all(_close(db64, _fd_grad(loss, b), 1.0))
    if weighted:
        assert np.all(_close(dw64, _fd_grad(loss, w), 1.0))


def test_glu_mag_bounds_the_gradient():
    r = rng(18)
    T, H = 32, 64
    x = bf16_bits(r.standard_normal((T, 2 * H)).astype(np.float32))
    g = bf16_bits(r.standard_normal((T, H)).astype(np.float32))
    for act in ("swiglu", "geglu"):
        _, d64, mag, _, _ = oracle.bias_glu_bwd(act, "bf16", g, x, None)
        assert np.all(mag * 2 >= np.abs(d64))


def test_glu_empty_tokens():
    x = np.zeros((0, 32), np.uint16)
    g = np.zeros((0, 16), np.uint16)
    _, _, _, db, dw = oracle.bias_glu_bwd("swiglu", "bf16", g, x, None, np.zeros(0, np.uint16))
    assert np.array_equal(db, np.zeros(32)) and dw.shape == (0,)


# ---------------------------------------------------------------- dropout-add backward

@pytest.mark.parametrize("p", [0.1, 0.5])
def test_bda_bwd_brute_force_jacobian(p):
    """Finite differences through the oracle's own train forward (double storage):
    d out / d x = keep * s, d out / d bias summed over rows, d out / d residual = 1."""
    r = rng(19)
    T, H, seed, off = 4, 8, 77, 3
    x = r.standard_normal((T, H))
    b = r.standard_normal(H) * 0.3
    res = r.standard_normal((T, H))
    g = r.standard_normal((T, H))
    dx, dx64, dres, db64 = oracle.bias_dropout_add_bwd("f64", g, "f64", p, seed, off)

    def loss():
        _, o, _ = oracle.bias_dropout_add("f64", x, b, res, "f64", True, p, seed, off)
        return float(np.sum(g * o))

    assert np.all(_close(dx64, _fd_grad(loss, x), 1.0))
    assert np.all(_close(db64, _fd_grad(loss, b), 1.0))
    assert np.all(_close(dres, _fd_grad(loss, res), 1.0))


def test_bda_bwd_follows_the_forward_mask_and_widens_the_residual_grad():
    T, H, p, seed, off = 16, 64, 0.3, 9, 2**32 + 1
    g = bf16_bits(rng(20).standard_normal((T, H)).astype(np.float32))
    dx, dx64, dres, db64 = oracle.bias_dropout_add_bwd("bf16", g, "f32", p, seed, off)
    bits = np.unpackbits(oracle.dropout_mask(T, H, p, seed, off), bitorder="little")[:T * H].reshape(T, H)
    s = float(np.float32(1.0 / (1.0 - float(np.float32(p)))))
    gv = bf16_value(g)
    assert np.array_equal(dx64, np.where(bits == 1, gv * s, 0.0))
    assert np.array_equal(dres.astype(np.float64), gv)       # bf16 -> fp32 is exact
    assert np.allclose(db64, dx64.sum(axis=0), rtol=1e-13, atol=1e-13)
    # row sampling gives the same rows
    dxp, *_ = oracle.bias_dropout_add_bwd("bf16", g[5:9], "f32", p, seed, off, row0=5)
    assert np.array_equal(dxp, dx[5:9])


def test_bda_bwd_p0_is_identity_and_p1_is_zero():
    g = bf16_bits(rng(21).standard_normal((8, 32)).astype(np.float32))
    dx, _, dres, db = oracle.bias_dropout_add_bwd("bf16", g, "bf16", 0.0, 1, 0)
    assert np.array_equal(dx, g) and np.array_equal(dres, g)
    dx1, d641, _, db1 = oracle.bias_dropout_add_bwd("bf16", g, "bf16", 1.0, 1, 0)
    assert np.all(d641 == 0.0) and np.all(db1 == 0.0)


# ---------------------------------------------------------------- exact (erf) GeLU ops

def test_gelu_erf_fwd_matches_torch_broadcast():
    r = rng(22)
    y = r.standard_normal((48, 72)).astype(np.float32) * 3
    b = (r.standard_normal(72) * 0.5).astype(np.float32)
    out, out64 = oracle.bias_gelu_fwd("f32", y, b, exact=True)
    z = torch.from_numpy(y).double() + torch.from_numpy(b).double()
    ref = F.gelu(z, approximate="none").numpy()
    # 0.70710678 vs 1/sqrt(2): 1.7e-9 relative in the argument, magnified ~z^2 in the tail
    tol = 2e-9 * (z.numpy() ** 2 + 2)
    assert np.all(np.abs(out64 - ref) <= tol * np.abs(ref) + 1e-15)
    assert np.array_equal(out, out64.astype(np.float32))


def test_gelu_erf_bwd_brute_force_jacobian_4x8():
    r = rng(23)
    y = r.standard_normal((4, 8)) * 2
    b = r.standard_normal(8) * 0.3
    g = r.standard_normal((4, 8))
    _, d64, mag, db64 = oracle.bias_gelu_bwd("f64", g, y, b, exact=True)

    def loss():
        _, o = oracle.bias_gelu_fwd("f64", y, b, exact=True)
        return float(np.sum(g * o))

    # the printed 0.3989423 and 0.70710678 agree to ~5e-8 (see the scalar pins)
    assert np.all(np.abs(d64 - _fd_grad(loss, y)) <= 1e-7 * np.abs(d64) + 5e-8)
    assert np.all(np.abs(db64 - _fd_grad(loss, b)) <= 1e-7 * np.abs(db64) + 5e-7)
    assert np.all(mag * 2 >= np.abs(d64))


def test_gelu_erf_differs_from_tanh_by_at_most_1e3():
    r = rng(24)
    y = (r.standard_normal((16, 64)) * 2).astype(np.float32)
    _, a = oracle.bias_gelu_fwd("f32", y, None)
    _, e = oracle.bias_gelu_fwd("f32", y, None, exact=True)
    d = np.abs(a - e)
    assert d.max() <= 1e-3 and d.max() > 1e-5
