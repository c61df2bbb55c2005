"""oracle32: the oracle's formulas evaluated in IEEE binary32 (oracle/oracle32.c).

TEST INFRASTRUCTURE ONLY (the test suite, the smoke check and the benchmark's
CPU-baseline leg). This is the plain fp32 scalar evaluation of each op: a
secondary statistic beside the fp64 parity reference (the functions of the
``oracle`` package) and the fp32 CPU baseline. It is not the parity reference.
The literal tanh GeLU derivative it evaluates cancels in float in the negative
tail, and its float row sums lose digits the fp64 oracle keeps.

Same array conventions as the ``oracle`` package: float32 storage for "f32",
uint16 bit patterns for "f16" / "bf16". Outputs are rounded once to their
dtype from the float value; gradient sums come back as float32 arrays.
"""
from __future__ import annotations

import numpy as np

from . import ACTS, DTYPES, _check_in, _ok, _ptr, _storage, lib

_D32 = {k: v for k, v in DTYPES.items() if k != "f64"}


def _dt(dt):
    if dt not in _D32:
        raise ValueError(f"oracle32 evaluates f32, f16 and bf16 storage, not {dt}")
    return _D32[dt]


def bias_gelu_fwd(dt, y, bias, exact=False):
    T, H = y.shape
    y = _check_in(y, dt, name="y")
    bias = _check_in(bias, dt, (H,), "bias")
    out = np.empty((T, H), _storage(dt))
    _ok(lib().orc32_bias_gelu_fwd(_dt(dt), int(bool(exact)), _ptr(y), _ptr(bias), _ptr(out), T, H))
    return out


def bias_gelu_bwd(dt, g, y, bias, exact=False):
    """Returns dgrad (dt storage), dbias (float32)."""
    T, H = y.shape
    y = _check_in(y, dt, name="y")
    g = _check_in(g, dt, (T, H), "g")
    bias = _check_in(bias, dt, (H,), "bias")
    dgrad = np.empty((T, H), _storage(dt))
    dbias = np.empty((H,), np.float32)
    _ok(lib().orc32_bias_gelu_bwd(_dt(dt), int(bool(exact)), _ptr(g), _ptr(y), _ptr(bias), _ptr(dgrad),
                                  _ptr(dbias), T, H))
    return dgrad, dbias


def bias_dropout_add(dt, x, bias, residual, res_dt, train, p=0.0, seed=0, offset=0, row0=0):
    T, H = x.shape
    x = _check_in(x, dt, name="x")
    bias = _check_in(bias, dt, (H,), "bias")
    residual = _check_in(residual, res_dt, (T, H), "residual")
    out = np.empty((T, H), _storage(dt))
    _ok(lib().orc32_bias_dropout_add(_dt(dt), _ptr(x), _ptr(bias), _ptr(residual), _dt(res_dt), _ptr(out), T, H,
                                     int(bool(train)), float(p), int(seed), int(offset), int(row0)))
    return out


def bias_dropout_add_bwd(dt, g, res_dt, p, seed, offset=0, row0=0, want_dres=True):
    """Returns dx (dt storage), dresidual (res_dt storage or None), dbias (float32)."""
    T, H = g.shape
    g = _check_in(g, dt, name="g")
    dx = np.empty((T, H), _storage(dt))
    dres = np.empty((T, H), _storage(res_dt)) if want_dres else None
    dbias = np.empty((H,), np.float32)
    _ok(lib().orc32_bias_dropout_add_bwd(_dt(dt), _ptr(g), _dt(res_dt), _ptr(dx), _ptr(dres), _ptr(dbias), T, H,
                                         float(p), int(seed), int(offset), int(row0)))
    return dx, dres, dbias


def bias_glu_fwd(act, dt, inp, bias, weights=None, w_dt=None):
    T, H2 = inp.shape
    H = H2 // 2
    inp = _check_in(inp, dt, name="in")
    bias = _check_in(bias, dt, (H2,), "bias")
    w_dt = w_dt or dt
    weights = _check_in(weights, w_dt, (T,), "weights")
    out = np.empty((T, H), _storage(dt))
    _ok(lib().orc32_bias_glu_fwd(ACTS[act], _dt(dt), _ptr(inp), _ptr(bias), _ptr(weights), _dt(w_dt), _ptr(out),
                                 T, H))
    return out


def bias_glu_bwd(act, dt, g, inp, bias, weights=None, w_dt=None):
    """Returns din (dt storage, [T, 2H]), dbias (float32 [2H]), dweights (float32 [T] or None)."""
    T, H2 = inp.shape
    H = H2 // 2
    inp = _check_in(inp, dt, name="in")
    g = _check_in(g, dt, (T, H), "g")
    bias = _check_in(bias, dt, (H2,), "bias")
    w_dt = w_dt or dt
    weights = _check_in(weights, w_dt, (T,), "weights")
    din = np.empty((T, H2), _storage(dt))
    dbias = np.empty((H2,), np.float32)
    dw = np.empty((T,), np.float32) if weights is not None else None
    _ok(lib().orc32_bias_glu_bwd(ACTS[act], _dt(dt), _ptr(g), _ptr(inp), _ptr(bias), _ptr(weights), _dt(w_dt),
                                 _ptr(din), _ptr(dbias), _ptr(dw), T, H))
    return din, dbias, dw


def add_layer_norm_fwd(dt, x, residual, res_dt, gamma, beta=None, eps=1e-5, zero_centered=False):
    """Returns h, y (dt storage), mean, rstd (float32 [T])."""
    T, H = x.shape
    x = _check_in(x, dt, name="x")
    residual = _check_in(residual, res_dt, (T, H), "residual")
    gamma = _check_in(gamma, dt, (H,), "gamma")
    beta = _check_in(beta, dt, (H,), "beta")
    h = np.empty((T, H), _storage(dt))
    y = np.empty((T, H), _storage(dt))
    mean = np.empty((T,), np.float32)
    rstd = np.empty((T,), np.float32)
    _ok(lib().orc32_add_layer_norm_fwd(_dt(dt), _ptr(x), _ptr(residual), _dt(res_dt), _ptr(gamma), _ptr(beta),
                                       int(bool(zero_centered)), float(eps), _ptr(h), _ptr(y), _ptr(mean),
                                       _ptr(rstd), T, H))
    return h, y, mean, rstd


def add_layer_norm_bwd(dt, dy, h, gamma, eps=1e-5, zero_centered=False, dh_in=None, res_dt=None, want_dres=True):
    """Returns dx (dt storage), dresidual (res_dt storage or None), dgamma, dbeta (float32 [H])."""
    T, H = h.shape
    res_dt = res_dt or dt
    dy = _check_in(dy, dt, (T, H), "dy")
    h = _check_in(h, dt, name="h")
    gamma = _check_in(gamma, dt, (H,), "gamma")
    dh_in = _check_in(dh_in, res_dt, (T, H), "dh_in")
    dx = np.empty((T, H), _storage(dt))
    dres = np.empty((T, H), _storage(res_dt)) if want_dres else None
    dgamma = np.empty((H,), np.float32)
    dbeta = np.empty((H,), np.float32)
    _ok(lib().orc32_add_layer_norm_bwd(_dt(dt), _ptr(dy), _ptr(h), _ptr(gamma), int(bool(zero_centered)),
                                       float(eps), _ptr(dh_in), _dt(res_dt), _ptr(dx), _ptr(dres), _ptr(dgamma),
                                       _ptr(dbeta), T, H))
    return dx, dres, dgamma, dbeta


def weighted_squared_relu_fwd(dt, x, weights=None, w_dt=None):
    T, H = x.shape
    x = _check_in(x, dt, name="x")
    w_dt = w_dt or dt
    weights = _check_in(weights, w_dt, (T,), "weights")
    out = np.empty((T, H), _storage(dt))
    _ok(lib().orc32_weighted_squared_relu_fwd(_dt(dt), _ptr(x), _ptr(weights), _dt(w_dt), _ptr(out), T, H))
    return out


def weighted_squared_relu_bwd(dt, g, x, weights=None, w_dt=None):
    """Returns dx (dt storage), dweights (float32 [T] or None)."""
    T, H = x.shape
    x = _check_in(x, dt, name="x")
    g = _check_in(g, dt, (T, H), "g")
    w_dt = w_dt or dt
    weights = _check_in(weights, w_dt, (T,), "weights")
    dx = np.empty((T, H), _storage(dt))
    dw = np.empty((T,), np.float32) if weights is not None else None
    _ok(lib().orc32_weighted_squared_relu_bwd(_dt(dt), _ptr(g), _ptr(x), _ptr(weights), _dt(w_dt), _ptr(dx),
                                              _ptr(dw), T, H))
    return dx, dw
