"""ctypes wrapper around the scalar CPU oracle (oracle/oracle.c).

TEST INFRASTRUCTURE ONLY: the test suite, the smoke check and the
benchmark's CPU-baseline leg are the only callers. The fused-epilogue
library never imports this package, and this package never imports the
library.

Arrays are numpy arrays holding the raw storage of a tensor: float32 for
``"f32"`` and uint16 bit patterns for ``"f16"`` / ``"bf16"``. Every function
returns the outputs rounded once to the output dtype (same raw storage
convention) together with the unrounded float64 values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_SRCS = [_SRC, os.path.join(_HERE, "oracle32.c")]  # oracle32.c: the same formulas in binary32
_LIB = os.path.join(_HERE, "liboracle.so")
_CFLAGS = ["-O2", "-std=c11", "-Wall", "-Wextra", "-ffp-contract=off", "-fno-fast-math", "-fPIC", "-shared"]

DTYPES = {"f32": 0, "f16": 1, "bf16": 2, "f64": 3}  # f64: oracle-only, for finite differences
ACTS = {"swiglu": 0, "geglu": 1}

_lock = threading.Lock()
_lib = None


def build(force: bool = False) -> str:
    """Compile liboracle.so with gcc (no fast-math, no FMA contraction)."""
    stale = not os.path.exists(_LIB) or any(os.path.getmtime(_LIB) < os.path.getmtime(f) for f in _SRCS)
    if force or stale:
        tmp = _LIB + ".tmp%d" % os.getpid()
        subprocess.run(["gcc", *_CFLAGS, *_SRCS, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


def lib() -> ctypes.CDLL:
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB)
            P, I64, I, D, F, U64 = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_double,
                                    ctypes.c_float, ctypes.c_uint64)
            L.orc_bias_gelu_fwd.argtypes = [I, P, P, P, P, I64, I64]
            L.orc_bias_gelu_bwd.argtypes = [I, P, P, P, P, P, P, P, I64, I64]
            L.orc_bias_gelu_erf_fwd.argtypes = [I, P, P, P, P, I64, I64]
            L.orc_bias_gelu_erf_bwd.argtypes = [I, P, P, P, P, P, P, P, I64, I64]
            L.orc_bias_dropout_add.argtypes = [I, P, P, P, I, P, P, P, I64, I64, I, F, U64, U64, I64]
            L.orc_dropout_mask.argtypes = [P, I64, I64, F, U64, U64, I64]
            L.orc_bias_dropout_add_bwd.argtypes = [I, P, I, P, P, P, P, I64, I64, F, U64, U64, I64]
            L.orc_bias_glu_fwd.argtypes = [I, I, P, P, P, I, P, P, I64, I64]
            L.orc_bias_glu_bwd.argtypes = [I, I, P, P, P, P, I, P, P, P, P, P, I64, I64]
            L.orc_add_layer_norm_fwd.argtypes = [I, P, P, I, P, P, I, F, P, P, P, P, P, P, I64, I64]
            L.orc_add_layer_norm_bwd.argtypes = [I, P, P, P, I, F, P, I, P, P, P, P, P, P, I64, I64]
            L.orc_weighted_squared_relu_fwd.argtypes = [I, P, P, I, P, P, I64, I64]
            L.orc_weighted_squared_relu_bwd.argtypes = [I, P, P, P, I, P, P, P, I64, I64]
            L.orc_philox4x32_10.argtypes = [P, P, P]
            L.orc_philox4x32_10.restype = None
            for name in ("orc_gelu_tanh", "orc_gelu_tanh_grad", "orc_gelu_erf", "orc_gelu_erf_grad",
                         "orc_silu", "orc_silu_grad"):
                getattr(L, name).argtypes = [D]
                getattr(L, name).restype = D
            L.orc_round_bf16.argtypes = [D]
            L.orc_round_bf16.restype = ctypes.c_uint16
            L.orc_round_f16.argtypes = [D]
            L.orc_round_f16.restype = ctypes.c_uint16
            L.orc_round_f32.argtypes = [D]
            L.orc_round_f32.restype = F
            L.orc_bf16_to_double.argtypes = [ctypes.c_uint16]
            L.orc_bf16_to_double.restype = D
            L.orc_f16_to_double.argtypes = [ctypes.c_uint16]
            L.orc_f16_to_double.restype = D
            L.orc_drop_threshold.argtypes = [F]
            L.orc_drop_threshold.restype = U64
            L.orc_keep_scale.argtypes = [F]
            L.orc_keep_scale.restype = F
            L.orc_decode.argtypes = [I, P, I64]
            L.orc_decode.restype = D
            # oracle32 (oracle32.c)
            L.orc32_bias_gelu_fwd.argtypes = [I, I, P, P, P, I64, I64]
            L.orc32_bias_gelu_bwd.argtypes = [I, I, P, P, P, P, P, I64, I64]
            L.orc32_bias_dropout_add.argtypes = [I, P, P, P, I, P, I64, I64, I, F, U64, U64, I64]
            L.orc32_bias_dropout_add_bwd.argtypes = [I, P, I, P, P, P, I64, I64, F, U64, U64, I64]
            L.orc32_bias_glu_fwd.argtypes = [I, I, P, P, P, I, P, I64, I64]
            L.orc32_bias_glu_bwd.argtypes = [I, I, P, P, P, P, I, P, P, P, I64, I64]
            L.orc32_add_layer_norm_fwd.argtypes = [I, P, P, I, P, P, I, F, P, P, P, P, I64, I64]
            L.orc32_add_layer_norm_bwd.argtypes = [I, P, P, P, I, F, P, I, P, P, P, P, I64, I64]
            L.orc32_weighted_squared_relu_fwd.argtypes = [I, P, P, I, P, I64, I64]
            L.orc32_weighted_squared_relu_bwd.argtypes = [I, P, P, P, I, P, P, I64, I64]
            _lib = L
    return _lib


def _storage(dt: str):
    return {"f32": np.float32, "f64": np.float64}.get(dt, np.uint16)


def _ptr(a):
    return None if a is None else a.ctypes.data


def _check_in(a, dt, shape=None, name="array"):
    if a is None:
        return None
    if a.dtype != _storage(dt):
        raise TypeError(f"{name}: storage {a.dtype} does not match dtype {dt}")
    if shape is not None and tuple(a.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {a.shape}, expected {shape}")
    return np.ascontiguousarray(a)


def _ok(rc):
    if rc != 0:
        raise ValueError("oracle rejected the arguments")


# --- scalar functions ------------------------------------------------------

def gelu_tanh(z: float) -> float:
    return lib().orc_gelu_tanh(float(z))


def gelu_tanh_grad(z: float) -> float:
    return lib().orc_gelu_tanh_grad(float(z))


def gelu_erf(z: float) -> float:
    return lib().orc_gelu_erf(float(z))


def gelu_erf_grad(z: float) -> float:
    return lib().orc_gelu_erf_grad(float(z))


def silu(a: float) -> float:
    return lib().orc_silu(float(a))


def silu_grad(a: float) -> float:
    return lib().orc_silu_grad(float(a))


def round_bf16(v: float) -> int:
    return int(lib().orc_round_bf16(float(v)))


def round_f16(v: float) -> int:
    return int(lib().orc_round_f16(float(v)))


def round_f32(v: float) -> float:
    return float(lib().orc_round_f32(float(v)))


def decode(dt: str, a: np.ndarray) -> np.ndarray:
    """Decode raw storage to float64 (elementwise, through the oracle's decoder)."""
    a = np.ascontiguousarray(a)
    if dt in ("f32", "f64"):
        return a.astype(np.float64)
    L = lib()
    f = L.orc_bf16_to_double if dt == "bf16" else L.orc_f16_to_double
    flat = a.reshape(-1)
    out = np.fromiter((f(int(v)) for v in flat), dtype=np.float64, count=flat.size)
    return out.reshape(a.shape)


def philox4x32_10(ctr, key):
    c = (ctypes.c_uint32 * 4)(*[int(v) & 0xFFFFFFFF for v in ctr])
    k = (ctypes.c_uint32 * 2)(*[int(v) & 0xFFFFFFFF for v in key])
    o = (ctypes.c_uint32 * 4)()
    lib().orc_philox4x32_10(c, k, o)
    return [int(v) for v in o]


def drop_threshold(p: float) -> int:
    return int(lib().orc_drop_threshold(float(p)))


def keep_scale(p: float) -> float:
    return float(lib().orc_keep_scale(float(p)))


# --- fused ops -------------------------------------------------------------

def bias_gelu_fwd(dt, y, bias, exact=False):
    """tanh-approximated GeLU, or the exact erf form with exact=True."""
    T, H = y.shape
    y = _check_in(y, dt, name="y")
    bias = _check_in(bias, dt, (H,), "bias")
    out = np.empty((T, H), _storage(dt))
    out64 = np.empty((T, H), np.float64)
    f = lib().orc_bias_gelu_erf_fwd if exact else lib().orc_bias_gelu_fwd
    _ok(f(DTYPES[dt], _ptr(y), _ptr(bias), _ptr(out), _ptr(out64), T, H))
    return out, out64


def bias_gelu_bwd(dt, g, y, bias, exact=False):
    """Returns dgrad (dt storage), dgrad64, mag64, dbias64."""
    T, H = y.shape
    y = _check_in(y, dt, name="y")
    g = _check_in(g, dt, (T, H), "g")
    bias = _check_in(bias, dt, (H,), "bias")
    dgrad = np.empty((T, H), _storage(dt))
    d64 = np.empty((T, H), np.float64)
    mag = np.empty((T, H), np.float64)
    dbias = np.empty((H,), np.float64)
    f = lib().orc_bias_gelu_erf_bwd if exact else lib().orc_bias_gelu_bwd
    _ok(f(DTYPES[dt], _ptr(g), _ptr(y), _ptr(bias), _ptr(dgrad), _ptr(d64), _ptr(mag), _ptr(dbias), T, H))
    return dgrad, d64, mag, dbias


def bias_dropout_add(dt, x, bias, residual, res_dt, train, p=0.0, seed=0, offset=0, row0=0):
    """Returns out (dt storage), out64, mag64."""
    T, H = x.shape
    x = _check_in(x, dt, name="x")
    bias = _check_in(bias, dt, (H,), "bias")
    residual = _check_in(residual, res_dt, (T, H), "residual")
    out = np.empty((T, H), _storage(dt))
    out64 = np.empty((T, H), np.float64)
    mag = np.empty((T, H), np.float64)
    _ok(lib().orc_bias_dropout_add(DTYPES[dt], _ptr(x), _ptr(bias), _ptr(residual), DTYPES[res_dt],
                                   _ptr(out), _ptr(out64), _ptr(mag), T, H, int(bool(train)),
                                   float(p), int(seed), int(offset), int(row0)))
    return out, out64, mag


def bias_dropout_add_bwd(dt, g, res_dt, p, seed, offset=0, row0=0, want_dres=True):
    """Returns dx (dt storage), dx64, dresidual (res_dt storage or None), dbias64."""
    T, H = g.shape
    g = _check_in(g, dt, name="g")
    dx = np.empty((T, H), _storage(dt))
    dx64 = np.empty((T, H), np.float64)
    dres = np.empty((T, H), _storage(res_dt)) if want_dres else None
    dbias = np.empty((H,), np.float64)
    _ok(lib().orc_bias_dropout_add_bwd(DTYPES[dt], _ptr(g), DTYPES[res_dt], _ptr(dx), _ptr(dx64), _ptr(dres),
                                       _ptr(dbias), T, H, float(p), int(seed), int(offset), int(row0)))
    return dx, dx64, dres, dbias


def add_layer_norm_fwd(dt, x, residual, res_dt, gamma, beta=None, eps=1e-5, zero_centered=False):
    """Residual add + LayerNorm. Returns h (dt storage), y (dt storage), y64,
    mag64, mean64 [T], rstd64 [T]."""
    T, H = x.shape
    x = _check_in(x, dt, name="x")
    residual = _check_in(residual, res_dt, (T, H), "residual")
    gamma = _check_in(gamma, dt, (H,), "gamma")
    beta = _check_in(beta, dt, (H,), "beta")
    h = np.empty((T, H), _storage(dt))
    y = np.empty((T, H), _storage(dt))
    y64 = np.empty((T, H), np.float64)
    mag = np.empty((T, H), np.float64)
    mean = np.empty((T,), np.float64)
    rstd = np.empty((T,), np.float64)
    _ok(lib().orc_add_layer_norm_fwd(DTYPES[dt], _ptr(x), _ptr(residual), DTYPES[res_dt], _ptr(gamma), _ptr(beta),
                                     int(bool(zero_centered)), float(eps), _ptr(h), _ptr(y), _ptr(y64), _ptr(mag),
                                     _ptr(mean), _ptr(rstd), T, H))
    return h, y, y64, mag, mean, rstd


def add_layer_norm_bwd(dt, dy, h, gamma, eps=1e-5, zero_centered=False, dh_in=None, res_dt=None,
                       want_dres=True):
    """Returns dx (dt storage), dx64, mag64, dresidual (res_dt storage or None),
    dgamma64 [H], dbeta64 [H]."""
    T, H = h.shape
    res_dt = res_dt or dt
    dy = _check_in(dy, dt, (T, H), "dy")
    h = _check_in(h, dt, name="h")
    gamma = _check_in(gamma, dt, (H,), "gamma")
    dh_in = _check_in(dh_in, res_dt, (T, H), "dh_in")
    dx = np.empty((T, H), _storage(dt))
    dx64 = np.empty((T, H), np.float64)
    mag = np.empty((T, H), np.float64)
    dres = np.empty((T, H), _storage(res_dt)) if want_dres else None
    dgamma = np.empty((H,), np.float64)
    dbeta = np.empty((H,), np.float64)
    _ok(lib().orc_add_layer_norm_bwd(DTYPES[dt], _ptr(dy), _ptr(h), _ptr(gamma), int(bool(zero_centered)),
                                     float(eps), _ptr(dh_in), DTYPES[res_dt], _ptr(dx), _ptr(dx64), _ptr(mag),
                                     _ptr(dres), _ptr(dgamma), _ptr(dbeta), T, H))
    return dx, dx64, mag, dres, dgamma, dbeta


def weighted_squared_relu_fwd(dt, x, weights=None, w_dt=None):
    """Returns out (dt storage), out64."""
    T, H = x.shape
    w_dt = w_dt or dt
    x = _check_in(x, dt, name="x")
    weights = _check_in(weights, w_dt, (T,), "weights")
    out = np.empty((T, H), _storage(dt))
    out64 = np.empty((T, H), np.float64)
    _ok(lib().orc_weighted_squared_relu_fwd(DTYPES[dt], _ptr(x), _ptr(weights), DTYPES[w_dt], _ptr(out), _ptr(out64),
                                            T, H))
    return out, out64


def weighted_squared_relu_bwd(dt, g, x, weights=None, w_dt=None):
    """Returns dx (dt storage), dx64, dweights64 [T] (None without weights)."""
    T, H = x.shape
    w_dt = w_dt or dt
    g = _check_in(g, dt, (T, H), "g")
    x = _check_in(x, dt, name="x")
    weights = _check_in(weights, w_dt, (T,), "weights")
    dx = np.empty((T, H), _storage(dt))
    dx64 = np.empty((T, H), np.float64)
    dw = np.empty((T,), np.float64) if weights is not None else None
    _ok(lib().orc_weighted_squared_relu_bwd(DTYPES[dt], _ptr(g), _ptr(x), _ptr(weights), DTYPES[w_dt], _ptr(dx),
                                            _ptr(dx64), _ptr(dw), T, H))
    return dx, dx64, dw


def dropout_mask(T, H, p, seed, offset, row0=0):
    """Keep bits, LSB-first by element index, as a uint8 array of ceil(T*H/8) bytes."""
    bits = np.empty(((T * H + 7) // 8,), np.uint8)
    _ok(lib().orc_dropout_mask(_ptr(bits), T, H, float(p), int(seed), int(offset), int(row0)))
    return bits


def bias_glu_fwd(act, dt, inp, bias, weights=None, w_dt=None):
    T, H2 = inp.shape
    H = H2 // 2
    if H2 != 2 * H:
        raise ValueError("gated input must have an even number of columns")
    w_dt = w_dt or dt
    inp = _check_in(inp, dt, name="in")
    bias = _check_in(bias, dt, (H2,), "bias")
    weights = _check_in(weights, w_dt, (T,), "weights")
    out = np.empty((T, H), _storage(dt))
    out64 = np.empty((T, H), np.float64)
    _ok(lib().orc_bias_glu_fwd(ACTS[act], DTYPES[dt], _ptr(inp), _ptr(bias), _ptr(weights),
                               DTYPES[w_dt], _ptr(out), _ptr(out64), T, H))
    return out, out64


def bias_glu_bwd(act, dt, g, inp, bias, weights=None, w_dt=None):
    """Returns din (dt storage), din64, mag64, dbias64 [2H], dweights64 [T] or None."""
    T, H2 = inp.shape
    H = H2 // 2
    w_dt = w_dt or dt
    inp = _check_in(inp, dt, name="in")
    g = _check_in(g, dt, (T, H), "g")
    bias = _check_in(bias, dt, (H2,), "bias")
    weights = _check_in(weights, w_dt, (T,), "weights")
    din = np.empty((T, H2), _storage(dt))
    d64 = np.empty((T, H2), np.float64)
    mag = np.empty((T, H2), np.float64)
    dbias = np.empty((H2,), np.float64)
    dw = np.empty((T,), np.float64) if weights is not None else None
    _ok(lib().orc_bias_glu_bwd(ACTS[act], DTYPES[dt], _ptr(g), _ptr(inp), _ptr(bias), _ptr(weights),
                               DTYPES[w_dt], _ptr(din), _ptr(d64), _ptr(mag), _ptr(dbias), _ptr(dw),
                               T, H))
    return din, d64, mag, dbias, dw
