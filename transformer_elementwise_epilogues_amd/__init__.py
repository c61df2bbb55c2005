"""Fused Transformer elementwise epilogues for AMD MI355X (gfx950).

Thin ctypes binding of ``libmb.so`` (C ABI in ``include/mb.h``): each
function takes torch CUDA tensors, passes their device pointers, shapes,
dtype and the current HIP stream to the ``mb_*`` entry point of the same
name, and raises :class:`MBError` on a non-zero status. All arithmetic runs
in the library's HIP kernels; torch only provides device memory and streams.
Outputs and workspaces the caller does not pass are allocated with torch.
"""
from __future__ import annotations

import ctypes
import os
import threading

import torch

__all__ = [
    "MBError", "lib", "abi_version",
    "mb_bias_gelu_fwd", "mb_bias_gelu_bwd", "mb_bias_gelu_bwd_workspace",
    "mb_bias_gelu_erf_fwd", "mb_bias_gelu_erf_bwd", "mb_bias_gelu_erf_bwd_workspace",
    "mb_bias_dropout_add_train", "mb_bias_dropout_add_infer", "mb_dropout_mask",
    "mb_bias_dropout_add_bwd", "mb_bias_dropout_add_bwd_workspace",
    "mb_bias_swiglu_fwd", "mb_bias_swiglu_bwd", "mb_bias_geglu_fwd", "mb_bias_geglu_bwd",
    "mb_bias_glu_bwd_workspace",
    "mb_add_layer_norm_fwd", "mb_add_layer_norm_bwd", "mb_add_layer_norm_bwd_workspace",
    "mb_weighted_squared_relu_fwd", "mb_weighted_squared_relu_bwd", "mb_weighted_squared_relu_bwd_workspace",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmb.so")
DTYPES = {torch.float32: 0, torch.float16: 1, torch.bfloat16: 2}

_lock = threading.Lock()
_lib = None


class MBError(RuntimeError):
    """A libmb entry point returned an error status."""

    def __init__(self, fn: str, status: int, message: str):
        super().__init__(f"{fn}: {message}")
        self.status = status


def lib() -> ctypes.CDLL:
    """Load libmb.so (built in-tree by ``build_lib``); fails loudly if it is missing."""
    global _lib
    with _lock:
        if _lib is None:
            if not os.path.exists(LIB_PATH):
                raise RuntimeError(f"{LIB_PATH} is not built: run `python -m "
                                   "transformer_elementwise_epilogues_amd.build_lib` (hipcc, gfx950)")
            L = ctypes.CDLL(LIB_PATH)
            P, I64, I, F, U64, SZ = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_float,
                                     ctypes.c_uint64, ctypes.c_size_t)
            sig = {
                "mb_status_string": ([I], ctypes.c_char_p),
                "mb_abi_version": ([], I),
                "mb_bias_gelu_fwd": ([P, P, P, I64, I64, I, P], I),
                "mb_bias_gelu_bwd_workspace": ([I64, I64, I, I], SZ),
                "mb_bias_gelu_bwd": ([P, P, P, P, P, P, SZ, I64, I64, I, P], I),
                "mb_bias_gelu_erf_fwd": ([P, P, P, I64, I64, I, P], I),
                "mb_bias_gelu_erf_bwd": ([P, P, P, P, P, P, SZ, I64, I64, I, P], I),
                "mb_bias_gelu_erf_bwd_workspace": ([I64, I64, I, I], SZ),
                "mb_bias_dropout_add_train": ([P, P, P, I, P, I64, I64, I, F, U64, U64, P], I),
                "mb_bias_dropout_add_infer": ([P, P, P, I, P, I64, I64, I, P], I),
                "mb_dropout_mask": ([P, I64, I64, F, U64, U64, P], I),
                "mb_bias_dropout_add_bwd_workspace": ([I64, I64, I, I], SZ),
                "mb_bias_dropout_add_bwd": ([P, P, P, I, P, P, SZ, I64, I64, I, F, U64, U64, P], I),
                "mb_bias_swiglu_fwd": ([P, P, P, I, P, I64, I64, I, P], I),
                "mb_bias_geglu_fwd": ([P, P, P, I64, I64, I, P], I),
                "mb_bias_glu_bwd_workspace": ([I64, I64, I, I, I], SZ),
                "mb_bias_swiglu_bwd": ([P, P, P, P, I, P, P, P, P, SZ, I64, I64, I, P], I),
                "mb_bias_geglu_bwd": ([P, P, P, P, P, P, SZ, I64, I64, I, P], I),
                "mb_add_layer_norm_fwd": ([P, P, I, P, P, F, I, P, P, P, P, I64, I64, I, P], I),
                "mb_add_layer_norm_bwd_workspace": ([I64, I64, I, I, I], SZ),
                "mb_weighted_squared_relu_fwd": ([P, P, I, P, I64, I64, I, P], I),
                "mb_weighted_squared_relu_bwd_workspace": ([I64, I64, I, I], SZ),
                "mb_weighted_squared_relu_bwd": ([P, P, P, I, P, P, P, SZ, I64, I64, I, P], I),
                "mb_add_layer_norm_bwd": ([P, P, P, P, P, I, P, I, P, P, P, P, P, SZ, I64, I64, I, P], I),
            }
            for name, (args, res) in sig.items():
                f = getattr(L, name)
                f.argtypes = args
                f.restype = res
            _lib = L
    return _lib


def abi_version() -> int:
    return lib().mb_abi_version()


def _p(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _dt(t: torch.Tensor) -> int:
    if t.dtype not in DTYPES:
        raise TypeError(f"unsupported dtype {t.dtype}")
    return DTYPES[t.dtype]


def _stream(t: torch.Tensor, stream):
    s = stream if stream is not None else torch.cuda.current_stream(t.device)
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn: str, status: int):
    if status != 0:
        raise MBError(fn, status, lib().mb_status_string(status).decode())


def _rows(t: torch.Tensor, name: str, cols=None):
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [tokens, hidden], got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if cols is not None and t.shape[1] != cols:
        raise ValueError(f"{name} has {t.shape[1]} columns, expected {cols}")
    return t.shape


def _vec(t, n, name):
    if t is None:
        return None
    if t.dim() != 1 or t.shape[0] != n or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous vector of {n} elements")
    return t


# ------------------------------------------------------------------ GeLU

def _gelu_fwd(fn, y, bias, out, stream):
    T, H = _rows(y, "y")
    _vec(bias, H, "bias")
    out = torch.empty_like(y) if out is None else out
    _check(fn, getattr(lib(), fn)(_p(y), _p(bias), _p(out), T, H, _dt(y), _stream(y, stream)))
    return out


def mb_bias_gelu_fwd(y, bias=None, out=None, stream=None):
    """tanh-approximated GeLU of y + bias; out=y runs in place."""
    return _gelu_fwd("mb_bias_gelu_fwd", y, bias, out, stream)


def mb_bias_gelu_erf_fwd(y, bias=None, out=None, stream=None):
    """Exact (erf) GeLU of y + bias; out=y runs in place."""
    return _gelu_fwd("mb_bias_gelu_erf_fwd", y, bias, out, stream)


def mb_bias_gelu_bwd_workspace(tokens, hidden, dtype, with_dbias=True) -> int:
    return int(lib().mb_bias_gelu_bwd_workspace(tokens, hidden, DTYPES[dtype], int(bool(with_dbias))))


def mb_bias_gelu_erf_bwd_workspace(tokens, hidden, dtype, with_dbias=True) -> int:
    return int(lib().mb_bias_gelu_erf_bwd_workspace(tokens, hidden, DTYPES[dtype], int(bool(with_dbias))))


def _gelu_bwd(fn, g, y, bias, dgrad, dbias, ws, stream):
    T, H = _rows(y, "y")
    _rows(g, "g", H)
    _vec(bias, H, "bias")
    dgrad = torch.empty_like(y) if dgrad is None else dgrad
    dbias = _grad_out(dbias, H, y.device)
    wsf = mb_bias_gelu_erf_bwd_workspace if fn == "mb_bias_gelu_erf_bwd" else mb_bias_gelu_bwd_workspace
    nws = wsf(T, H, y.dtype, dbias is not None)
    if ws is None and nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=y.device)
    _check(fn, getattr(lib(), fn)(_p(g), _p(y), _p(bias), _p(dgrad), _p(dbias), _p(ws),
                                  ws.numel() if ws is not None else 0, T, H, _dt(y), _stream(y, stream)))
    return dgrad, dbias


def mb_bias_gelu_bwd(g, y, bias=None, dgrad=None, dbias=True, ws=None, stream=None):
    """Returns (dgrad, dbias or None). dbias=True allocates the fp32 bias gradient."""
    return _gelu_bwd("mb_bias_gelu_bwd", g, y, bias, dgrad, dbias, ws, stream)


def mb_bias_gelu_erf_bwd(g, y, bias=None, dgrad=None, dbias=True, ws=None, stream=None):
    """Backward of the exact (erf) GeLU; returns (dgrad, dbias or None)."""
    return _gelu_bwd("mb_bias_gelu_erf_bwd", g, y, bias, dgrad, dbias, ws, stream)


# ------------------------------------------------------------------ dropout-add

def mb_bias_dropout_add_train(x, bias, residual, p, seed, offset=0, out=None, stream=None):
    T, H = _rows(x, "x")
    _rows(residual, "residual", H)
    _vec(bias, H, "bias")
    out = torch.empty_like(x) if out is None else out
    _check("mb_bias_dropout_add_train", lib().mb_bias_dropout_add_train(
        _p(x), _p(bias), _p(residual), _dt(residual), _p(out), T, H, _dt(x), float(p), int(seed), int(offset),
        _stream(x, stream)))
    return out


def mb_bias_dropout_add_infer(x, bias, residual, out=None, stream=None):
    """out=x runs in place."""
    T, H = _rows(x, "x")
    _rows(residual, "residual", H)
    _vec(bias, H, "bias")
    out = torch.empty_like(x) if out is None else out
    _check("mb_bias_dropout_add_infer", lib().mb_bias_dropout_add_infer(
        _p(x), _p(bias), _p(residual), _dt(residual), _p(out), T, H, _dt(x), _stream(x, stream)))
    return out


def mb_bias_dropout_add_bwd_workspace(tokens, hidden, dtype, with_dbias=True) -> int:
    return int(lib().mb_bias_dropout_add_bwd_workspace(tokens, hidden, DTYPES[dtype], int(bool(with_dbias))))


def mb_bias_dropout_add_bwd(g, p, seed, offset=0, residual_dtype=None, dx=None, dresidual=True, dbias=True,
                            ws=None, stream=None):
    """Returns (dx, dresidual or None, dbias or None) for the train forward with (p, seed, offset).
    residual_dtype defaults to g's dtype; dresidual=True allocates it, False skips it."""
    T, H = _rows(g, "g")
    rdt = residual_dtype or g.dtype
    dx = torch.empty_like(g) if dx is None else dx
    if dresidual is True:
        dresidual = torch.empty((T, H), dtype=rdt, device=g.device)
    elif dresidual is False:
        dresidual = None
    dbias = _grad_out(dbias, H, g.device)
    nws = mb_bias_dropout_add_bwd_workspace(T, H, g.dtype, dbias is not None)
    if ws is None and nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=g.device)
    _check("mb_bias_dropout_add_bwd", lib().mb_bias_dropout_add_bwd(
        _p(g), _p(dx), _p(dresidual), DTYPES[rdt], _p(dbias), _p(ws), ws.numel() if ws is not None else 0, T, H,
        _dt(g), float(p), int(seed), int(offset), _stream(g, stream)))
    return dx, dresidual, dbias


def mb_dropout_mask(tokens, hidden, p, seed, offset=0, device="cuda", out=None, stream=None):
    nbytes = (tokens * hidden + 7) // 8
    out = torch.empty(nbytes, dtype=torch.uint8, device=device) if out is None else out
    _check("mb_dropout_mask", lib().mb_dropout_mask(_p(out), tokens, hidden, float(p), int(seed), int(offset),
                                                    _stream(out, stream)))
    return out


# ------------------------------------------------------------------ gated units

def _glu_shapes(inp):
    T, H2 = _rows(inp, "in")
    if H2 % 2:
        raise ValueError("gated input needs an even number of columns")
    return T, H2 // 2


def mb_bias_swiglu_fwd(inp, bias=None, weights=None, out=None, stream=None):
    T, H = _glu_shapes(inp)
    _vec(bias, 2 * H, "bias")
    _vec(weights, T, "weights")
    out = torch.empty((T, H), dtype=inp.dtype, device=inp.device) if out is None else out
    wdt = _dt(weights) if weights is not None else _dt(inp)
    _check("mb_bias_swiglu_fwd", lib().mb_bias_swiglu_fwd(
        _p(inp), _p(bias), _p(weights), wdt, _p(out), T, H, _dt(inp), _stream(inp, stream)))
    return out


def mb_bias_geglu_fwd(inp, bias=None, out=None, stream=None):
    T, H = _glu_shapes(inp)
    _vec(bias, 2 * H, "bias")
    out = torch.empty((T, H), dtype=inp.dtype, device=inp.device) if out is None else out
    _check("mb_bias_geglu_fwd", lib().mb_bias_geglu_fwd(_p(inp), _p(bias), _p(out), T, H, _dt(inp),
                                                        _stream(inp, stream)))
    return out


def mb_bias_glu_bwd_workspace(tokens, hidden, dtype, with_dbias=True, with_dweights=False) -> int:
    return int(lib().mb_bias_glu_bwd_workspace(tokens, hidden, DTYPES[dtype], int(bool(with_dbias)),
                                               int(bool(with_dweights))))


def _grad_out(flag, n, device):
    if flag is True:
        return torch.empty(n, dtype=torch.float32, device=device)
    return None if flag is False or flag is None else flag


def mb_bias_swiglu_bwd(g, inp, bias=None, weights=None, din=None, dbias=True, dweights=None, ws=None,
                       stream=None):
    """Returns (din, dbias or None, dweights or None). dweights defaults to True when weights are given."""
    T, H = _glu_shapes(inp)
    _rows(g, "g", H)
    _vec(bias, 2 * H, "bias")
    _vec(weights, T, "weights")
    if dweights is None:
        dweights = weights is not None
    din = torch.empty_like(inp) if din is None else din
    dbias = _grad_out(dbias, 2 * H, inp.device)
    dweights = _grad_out(dweights, T, inp.device)
    nws = mb_bias_glu_bwd_workspace(T, H, inp.dtype, dbias is not None, dweights is not None)
    if ws is None and nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=inp.device)
    wdt = _dt(weights) if weights is not None else _dt(inp)
    _check("mb_bias_swiglu_bwd", lib().mb_bias_swiglu_bwd(
        _p(g), _p(inp), _p(bias), _p(weights), wdt, _p(din), _p(dbias), _p(dweights), _p(ws),
        ws.numel() if ws is not None else 0, T, H, _dt(inp), _stream(inp, stream)))
    return din, dbias, dweights


def mb_bias_geglu_bwd(g, inp, bias=None, din=None, dbias=True, ws=None, stream=None):
    """Returns (din, dbias or None)."""
    T, H = _glu_shapes(inp)
    _rows(g, "g", H)
    _vec(bias, 2 * H, "bias")
    din = torch.empty_like(inp) if din is None else din
    dbias = _grad_out(dbias, 2 * H, inp.device)
    nws = mb_bias_glu_bwd_workspace(T, H, inp.dtype, dbias is not None, False)
    if ws is None and nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=inp.device)
    _check("mb_bias_geglu_bwd", lib().mb_bias_geglu_bwd(
        _p(g), _p(inp), _p(bias), _p(din), _p(dbias), _p(ws), ws.numel() if ws is not None else 0, T, H,
        _dt(inp), _stream(inp, stream)))
    return din, dbias


# ------------------------------------------------------------------ residual add + LayerNorm

def mb_add_layer_norm_fwd(x, residual, gamma, beta=None, eps=1e-5, zero_centered_gamma=False, h_out=True,
                          y=None, stats=True, stream=None):
    """h = x + residual (cast to x's dtype), y = LayerNorm(h) * gamma' + beta.
    Returns (y, h or None, mean or None, rstd or None). h_out=True allocates h
    (False skips it; a tensor, e.g. x itself, receives it); stats=True
    allocates the fp32 mean / rstd the backward needs (or pass the pair)."""
    T, H = _rows(x, "x")
    _rows(residual, "residual", H)
    if residual.shape[0] != T:
        raise ValueError("residual must have x's shape")
    _vec(gamma, H, "gamma")
    _vec(beta, H, "beta")
    if h_out is True:
        h_out = torch.empty_like(x)
    elif h_out is False:
        h_out = None
    y = torch.empty_like(x) if y is None else y
    mean = rstd = None
    if stats is True:
        mean = torch.empty(T, dtype=torch.float32, device=x.device)
        rstd = torch.empty(T, dtype=torch.float32, device=x.device)
    elif stats:
        mean, rstd = stats
        _vec(mean, T, "mean")
        _vec(rstd, T, "rstd")
    _check("mb_add_layer_norm_fwd", lib().mb_add_layer_norm_fwd(
        _p(x), _p(residual), _dt(residual), _p(gamma), _p(beta), float(eps), int(bool(zero_centered_gamma)),
        _p(h_out), _p(y), _p(mean), _p(rstd), T, H, _dt(x), _stream(x, stream)))
    return y, h_out, mean, rstd


def mb_add_layer_norm_bwd_workspace(tokens, hidden, dtype, residual_dtype=None, with_param_grads=True) -> int:
    rdt = residual_dtype or dtype
    return int(lib().mb_add_layer_norm_bwd_workspace(tokens, hidden, DTYPES[dtype], DTYPES[rdt],
                                                     int(bool(with_param_grads))))


def mb_add_layer_norm_bwd(dy, h, gamma, mean, rstd, zero_centered_gamma=False, dh_in=None, residual_dtype=None,
                          dx=None, dresidual=False, dgamma=True, dbeta=True, ws=None, stream=None):
    """Returns (dx, dresidual or None, dgamma or None, dbeta or None).
    residual_dtype (default: dh_in's dtype, else h's) is the dtype of dh_in and
    dresidual; dresidual=True allocates it."""
    T, H = _rows(h, "h")
    _rows(dy, "dy", H)
    _vec(gamma, H, "gamma")
    _vec(mean, T, "mean")
    _vec(rstd, T, "rstd")
    rdt = residual_dtype or (dh_in.dtype if dh_in is not None else h.dtype)
    if dh_in is not None:
        _rows(dh_in, "dh_in", H)
    dx = torch.empty_like(h) if dx is None else dx
    if dresidual is True:
        dresidual = torch.empty((T, H), dtype=rdt, device=h.device)
    elif dresidual is False:
        dresidual = None
    dgamma = _grad_out(dgamma, H, h.device)
    dbeta = _grad_out(dbeta, H, h.device)
    nws = mb_add_layer_norm_bwd_workspace(T, H, h.dtype, rdt, dgamma is not None or dbeta is not None)
    if ws is None and nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=h.device)
    _check("mb_add_layer_norm_bwd", lib().mb_add_layer_norm_bwd(
        _p(dy), _p(h), _p(gamma), _p(mean), _p(rstd), int(bool(zero_centered_gamma)), _p(dh_in), DTYPES[rdt],
        _p(dx), _p(dresidual), _p(dgamma), _p(dbeta), _p(ws), ws.numel() if ws is not None else 0, T, H,
        _dt(h), _stream(h, stream)))
    return dx, dresidual, dgamma, dbeta


# ------------------------------------------------------------------ weighted squared ReLU

def mb_weighted_squared_relu_fwd(x, weights=None, out=None, stream=None):
    """relu(x)^2 * weights[t] (weights None: the plain squared ReLU); out=x runs in place."""
    T, H = _rows(x, "x")
    _vec(weights, T, "weights")
    out = torch.empty_like(x) if out is None else out
    wdt = _dt(weights) if weights is not None else 0
    _check("mb_weighted_squared_relu_fwd", lib().mb_weighted_squared_relu_fwd(
        _p(x), _p(weights), wdt, _p(out), T, H, _dt(x), _stream(x, stream)))
    return out


def mb_weighted_squared_relu_bwd_workspace(tokens, hidden, dtype, with_dweights=True) -> int:
    return int(lib().mb_weighted_squared_relu_bwd_workspace(tokens, hidden, DTYPES[dtype], int(bool(with_dweights))))


def mb_weighted_squared_relu_bwd(g, x, weights=None, dx=None, dweights=None, ws=None, stream=None):
    """Returns (dx, dweights or None); dweights defaults to True when weights are given."""
    T, H = _rows(x, "x")
    _rows(g, "g", H)
    _vec(weights, T, "weights")
    if dweights is None:
        dweights = weights is not None
    dx = torch.empty_like(x) if dx is None else dx
    dweights = _grad_out(dweights, T, x.device)
    nws = mb_weighted_squared_relu_bwd_workspace(T, H, x.dtype, dweights is not None)
    if ws is None and nws:
        ws = torch.empty(nws, dtype=torch.uint8, device=x.device)
    wdt = _dt(weights) if weights is not None else 0
    _check("mb_weighted_squared_relu_bwd", lib().mb_weighted_squared_relu_bwd(
        _p(g), _p(x), _p(weights), wdt, _p(dx), _p(dweights), _p(ws), ws.numel() if ws is not None else 0, T, H,
        _dt(x), _stream(x, stream)))
    return dx, dweights
