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
    "mb_bias_gelu_fwd", "mb_bias_gelu_bwd", "mb_bias_gelu_bwd_workspace", "mb_bias_gelu_bwd_noalloc",
    "mb_bias_gelu_erf_fwd", "mb_bias_gelu_erf_bwd", "mb_bias_gelu_erf_bwd_workspace",
    "mb_bias_dropout_add_train", "mb_bias_dropout_add_infer", "mb_dropout_mask",
    "mb_bias_dropout_add_bwd", "mb_bias_dropout_add_bwd_workspace",
    "mb_bias_swiglu_fwd", "mb_bias_swiglu_bwd", "mb_bias_geglu_fwd", "mb_bias_geglu_bwd",
    "mb_bias_glu_bwd_workspace",
    "mb_add_layer_norm_fwd", "mb_add_layer_norm_bwd", "mb_add_layer_norm_bwd_workspace",
    "mb_weighted_squared_relu_fwd", "mb_weighted_squared_relu_bwd", "mb_weighted_squared_relu_bwd_workspace",
    "mb_set_layer_norm_team_wait",
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
                "mb_bias_gelu_bwd_noalloc": ([P, P, P, P, P, I64, I64, I, P], I),
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
                "mb_set_layer_norm_team_wait": ([I], None),
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
        raise ValueError(f"unsupported dtype {t.dtype}")
    return DTYPES[t.dtype]


def _check(fn: str, status: int):
    if status != 0:
        raise MBError(fn, status, lib().mb_status_string(status).decode())


# Argument checks. The C ABI receives raw pointers and (tokens, hidden) only,
# so every size, dtype and device rule that a pointer alone cannot carry is
# enforced here, before any library call: each tensor argument, input or
# output, must have exactly the shape the entry point reads or writes, an
# accepted dtype, a contiguous layout, and live on the same GPU as the others
# (a host address handed to a kernel would fault the device). What the ABI
# checks itself from the pointers (alignment, overlap, the 16-byte row rule,
# the workspace size) is left to it.

def _need(t, name: str, shape, dtypes):
    """Check one tensor argument (not yet its device)."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")
    if t.dtype not in dtypes:
        names = ", ".join(str(d) for d in dtypes)
        raise ValueError(f"{name} has dtype {t.dtype}, expected {names}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t


def _opt(t, name: str, shape, dtypes):
    return None if t is None else _need(t, name, shape, dtypes)


def _rows2d(t, name: str):
    """[tokens, columns] of the tensor that defines an op's shape."""
    if not isinstance(t, torch.Tensor):
        raise ValueError(f"{name} must be a torch.Tensor, got {type(t).__name__}")
    if t.dim() != 2:
        raise ValueError(f"{name} must be 2-D [tokens, hidden], got {tuple(t.shape)}")
    if t.dtype not in DTYPES:
        raise ValueError(f"{name} has unsupported dtype {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.shape


def _gpu(stream, *named):
    """All (name, tensor) pairs (None skipped) on one GPU; `stream`, if given,
    on that GPU too. Returns the device."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if not t.is_cuda:
            raise ValueError(f"{name} must be a GPU tensor, got one on {t.device}")
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, the other tensors on {dev}")
    if stream is not None and dev is not None and torch.device(stream.device) != dev:
        raise ValueError(f"stream is on {stream.device}, the tensors on {dev}")
    return dev


def _stream(dev, stream):
    s = stream if stream is not None else torch.cuda.current_stream(dev)
    return ctypes.c_void_p(s.cuda_stream)


def _on(dev, name: str, t):
    """A caller-supplied output or buffer on the inputs' GPU."""
    if not t.is_cuda or t.device != dev:
        raise ValueError(f"{name} is on {t.device}, the inputs on {dev}")
    return t


def _out(t, name: str, shape, dtype, dev):
    """An output: allocated when not given, else checked like an input."""
    if t is None:
        return torch.empty(shape, dtype=dtype, device=dev)
    return _on(dev, name, _need(t, name, shape, (dtype,)))


def _grad_out(flag, name: str, n: int, dev):
    """An optional fp32 gradient vector: True allocates it, False/None skips it."""
    if flag is True:
        return torch.empty(n, dtype=torch.float32, device=dev)
    if flag is False or flag is None:
        return None
    return _on(dev, name, _need(flag, name, (n,), (torch.float32,)))


def _ws(ws, nbytes: int, dev):
    """The workspace: allocated when not given (nbytes > 0), else a contiguous
    tensor on the GPU; its byte size goes to the ABI, which checks it."""
    if ws is None:
        return (torch.empty(nbytes, dtype=torch.uint8, device=dev) if nbytes else None), nbytes
    if not isinstance(ws, torch.Tensor) or not ws.is_contiguous():
        raise ValueError("ws must be a contiguous torch.Tensor")
    return _on(dev, "ws", ws), ws.numel() * ws.element_size()


_FLOAT = tuple(DTYPES)


# ------------------------------------------------------------------ GeLU

def _gelu_fwd(fn, y, bias, out, stream):
    T, H = _rows2d(y, "y")
    _opt(bias, "bias", (H,), (y.dtype,))
    dev = _gpu(stream, ("y", y), ("bias", bias))
    out = _out(out, "out", (T, H), y.dtype, dev)
    _check(fn, getattr(lib(), fn)(_p(y), _p(bias), _p(out), T, H, _dt(y), _stream(dev, stream)))
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


def _gelu_bwd_args(g, y, bias, dgrad, dbias, stream):
    T, H = _rows2d(y, "y")
    _need(g, "g", (T, H), (y.dtype,))
    _opt(bias, "bias", (H,), (y.dtype,))
    dev = _gpu(stream, ("y", y), ("g", g), ("bias", bias))
    return T, H, dev, _out(dgrad, "dgrad", (T, H), y.dtype, dev), _grad_out(dbias, "dbias", H, dev)


def _gelu_bwd(fn, g, y, bias, dgrad, dbias, ws, stream):
    T, H, dev, dgrad, dbias = _gelu_bwd_args(g, y, bias, dgrad, dbias, stream)
    wsf = mb_bias_gelu_erf_bwd_workspace if fn == "mb_bias_gelu_erf_bwd" else mb_bias_gelu_bwd_workspace
    ws, nws = _ws(ws, wsf(T, H, y.dtype, dbias is not None), dev)
    _check(fn, getattr(lib(), fn)(_p(g), _p(y), _p(bias), _p(dgrad), _p(dbias), _p(ws), nws, T, H, _dt(y),
                                  _stream(dev, stream)))
    return dgrad, dbias


def mb_bias_gelu_bwd(g, y, bias=None, dgrad=None, dbias=True, ws=None, stream=None):
    """Returns (dgrad, dbias or None). dbias=True allocates the fp32 bias gradient."""
    return _gelu_bwd("mb_bias_gelu_bwd", g, y, bias, dgrad, dbias, ws, stream)


def mb_bias_gelu_erf_bwd(g, y, bias=None, dgrad=None, dbias=True, ws=None, stream=None):
    """Backward of the exact (erf) GeLU; returns (dgrad, dbias or None)."""
    return _gelu_bwd("mb_bias_gelu_erf_bwd", g, y, bias, dgrad, dbias, ws, stream)


def mb_bias_gelu_bwd_noalloc(g, y, bias=None, dgrad=None, dbias=True, stream=None):
    """mb_bias_gelu_bwd without a workspace: the library's static device
    scratch holds the bias gradient's partial rows (the C entry point
    allocates nothing; outputs not passed here are still allocated by torch).
    Returns (dgrad, dbias or None)."""
    T, H, dev, dgrad, dbias = _gelu_bwd_args(g, y, bias, dgrad, dbias, stream)
    _check("mb_bias_gelu_bwd_noalloc", lib().mb_bias_gelu_bwd_noalloc(
        _p(g), _p(y), _p(bias), _p(dgrad), _p(dbias), T, H, _dt(y), _stream(dev, stream)))
    return dgrad, dbias


# ------------------------------------------------------------------ dropout-add

def _res_dtypes(x):
    return (x.dtype, torch.float32)


def mb_bias_dropout_add_train(x, bias, residual, p, seed, offset=0, out=None, stream=None):
    """out = residual' + dropout(x + bias) with the Philox keep mask of (p, seed, offset)."""
    T, H = _rows2d(x, "x")
    _need(residual, "residual", (T, H), _res_dtypes(x))
    _opt(bias, "bias", (H,), (x.dtype,))
    dev = _gpu(stream, ("x", x), ("residual", residual), ("bias", bias))
    out = _out(out, "out", (T, H), x.dtype, dev)
    _check("mb_bias_dropout_add_train", lib().mb_bias_dropout_add_train(
        _p(x), _p(bias), _p(residual), _dt(residual), _p(out), T, H, _dt(x), float(p), int(seed), int(offset),
        _stream(dev, stream)))
    return out


def mb_bias_dropout_add_infer(x, bias, residual, out=None, stream=None):
    """out = residual' + x + bias; out=x runs in place."""
    T, H = _rows2d(x, "x")
    _need(residual, "residual", (T, H), _res_dtypes(x))
    _opt(bias, "bias", (H,), (x.dtype,))
    dev = _gpu(stream, ("x", x), ("residual", residual), ("bias", bias))
    out = _out(out, "out", (T, H), x.dtype, dev)
    _check("mb_bias_dropout_add_infer", lib().mb_bias_dropout_add_infer(
        _p(x), _p(bias), _p(residual), _dt(residual), _p(out), T, H, _dt(x), _stream(dev, stream)))
    return out


def mb_bias_dropout_add_bwd_workspace(tokens, hidden, dtype, with_dbias=True) -> int:
    return int(lib().mb_bias_dropout_add_bwd_workspace(tokens, hidden, DTYPES[dtype], int(bool(with_dbias))))


def mb_bias_dropout_add_bwd(g, p, seed, offset=0, residual_dtype=None, dx=None, dresidual=True, dbias=True,
                            ws=None, stream=None):
    """Returns (dx, dresidual or None, dbias or None) for the train forward with (p, seed, offset).
    residual_dtype defaults to g's dtype; dresidual=True allocates it, False skips it."""
    T, H = _rows2d(g, "g")
    rdt = residual_dtype or g.dtype
    if rdt not in _res_dtypes(g):
        raise ValueError(f"residual_dtype must be {g.dtype} or torch.float32, got {rdt}")
    dev = _gpu(stream, ("g", g))
    dx = _out(dx, "dx", (T, H), g.dtype, dev)
    if dresidual is True:
        dresidual = torch.empty((T, H), dtype=rdt, device=dev)
    elif dresidual is False or dresidual is None:
        dresidual = None
    else:
        _on(dev, "dresidual", _need(dresidual, "dresidual", (T, H), (rdt,)))
    dbias = _grad_out(dbias, "dbias", H, dev)
    ws, nws = _ws(ws, mb_bias_dropout_add_bwd_workspace(T, H, g.dtype, dbias is not None), dev)
    _check("mb_bias_dropout_add_bwd", lib().mb_bias_dropout_add_bwd(
        _p(g), _p(dx), _p(dresidual), DTYPES[rdt], _p(dbias), _p(ws), nws, T, H, _dt(g), float(p), int(seed),
        int(offset), _stream(dev, stream)))
    return dx, dresidual, dbias


def mb_dropout_mask(tokens, hidden, p, seed, offset=0, device="cuda", out=None, stream=None):
    """The keep bits of (tokens, hidden, p, seed, offset), LSB-first by element index."""
    nbytes = (tokens * hidden + 7) // 8
    if out is None:
        dev = torch.device(device)
        if dev.type != "cuda":
            raise ValueError(f"the mask is computed on a GPU, not on {dev}")
        out = torch.empty(nbytes, dtype=torch.uint8, device=dev)
    _need(out, "out", (nbytes,), (torch.uint8,))
    dev = _gpu(stream, ("out", out))
    _check("mb_dropout_mask", lib().mb_dropout_mask(_p(out), tokens, hidden, float(p), int(seed), int(offset),
                                                    _stream(dev, stream)))
    return out


# ------------------------------------------------------------------ gated units

def _glu_shapes(inp):
    T, H2 = _rows2d(inp, "in")
    if H2 % 2:
        raise ValueError("gated input needs an even number of columns")
    return T, H2 // 2


def _weights_dtype(weights, inp):
    return _dt(weights) if weights is not None else _dt(inp)


def mb_bias_swiglu_fwd(inp, bias=None, weights=None, out=None, stream=None):
    """silu(a) * b (* weights[t]) of the split input row plus bias."""
    T, H = _glu_shapes(inp)
    _opt(bias, "bias", (2 * H,), (inp.dtype,))
    _opt(weights, "weights", (T,), (inp.dtype, torch.float32))
    dev = _gpu(stream, ("in", inp), ("bias", bias), ("weights", weights))
    out = _out(out, "out", (T, H), inp.dtype, dev)
    _check("mb_bias_swiglu_fwd", lib().mb_bias_swiglu_fwd(
        _p(inp), _p(bias), _p(weights), _weights_dtype(weights, inp), _p(out), T, H, _dt(inp),
        _stream(dev, stream)))
    return out


def mb_bias_geglu_fwd(inp, bias=None, out=None, stream=None):
    """gelu_tanh(a) * b of the split input row plus bias."""
    T, H = _glu_shapes(inp)
    _opt(bias, "bias", (2 * H,), (inp.dtype,))
    dev = _gpu(stream, ("in", inp), ("bias", bias))
    out = _out(out, "out", (T, H), inp.dtype, dev)
    _check("mb_bias_geglu_fwd", lib().mb_bias_geglu_fwd(_p(inp), _p(bias), _p(out), T, H, _dt(inp),
                                                        _stream(dev, stream)))
    return out


def mb_bias_glu_bwd_workspace(tokens, hidden, dtype, with_dbias=True, with_dweights=False) -> int:
    return int(lib().mb_bias_glu_bwd_workspace(tokens, hidden, DTYPES[dtype], int(bool(with_dbias)),
                                               int(bool(with_dweights))))


def mb_bias_swiglu_bwd(g, inp, bias=None, weights=None, din=None, dbias=True, dweights=None, ws=None,
                       stream=None):
    """Returns (din, dbias or None, dweights or None). dweights defaults to True when weights are given."""
    T, H = _glu_shapes(inp)
    _need(g, "g", (T, H), (inp.dtype,))
    _opt(bias, "bias", (2 * H,), (inp.dtype,))
    _opt(weights, "weights", (T,), (inp.dtype, torch.float32))
    dev = _gpu(stream, ("in", inp), ("g", g), ("bias", bias), ("weights", weights))
    if dweights is None:
        dweights = weights is not None
    din = _out(din, "din", (T, 2 * H), inp.dtype, dev)
    dbias = _grad_out(dbias, "dbias", 2 * H, dev)
    dweights = _grad_out(dweights, "dweights", T, dev)
    ws, nws = _ws(ws, mb_bias_glu_bwd_workspace(T, H, inp.dtype, dbias is not None, dweights is not None), dev)
    _check("mb_bias_swiglu_bwd", lib().mb_bias_swiglu_bwd(
        _p(g), _p(inp), _p(bias), _p(weights), _weights_dtype(weights, inp), _p(din), _p(dbias), _p(dweights),
        _p(ws), nws, T, H, _dt(inp), _stream(dev, stream)))
    return din, dbias, dweights


def mb_bias_geglu_bwd(g, inp, bias=None, din=None, dbias=True, ws=None, stream=None):
    """Returns (din, dbias or None)."""
    T, H = _glu_shapes(inp)
    _need(g, "g", (T, H), (inp.dtype,))
    _opt(bias, "bias", (2 * H,), (inp.dtype,))
    dev = _gpu(stream, ("in", inp), ("g", g), ("bias", bias))
    din = _out(din, "din", (T, 2 * H), inp.dtype, dev)
    dbias = _grad_out(dbias, "dbias", 2 * H, dev)
    ws, nws = _ws(ws, mb_bias_glu_bwd_workspace(T, H, inp.dtype, dbias is not None, False), dev)
    _check("mb_bias_geglu_bwd", lib().mb_bias_geglu_bwd(
        _p(g), _p(inp), _p(bias), _p(din), _p(dbias), _p(ws), nws, T, H, _dt(inp), _stream(dev, stream)))
    return din, dbias


# ------------------------------------------------------------------ residual add + LayerNorm

def mb_add_layer_norm_fwd(x, residual, gamma, beta=None, eps=1e-5, zero_centered_gamma=False, h_out=True,
                          y=None, stats=True, stream=None):
    """h = x + residual (cast to x's dtype), y = LayerNorm(h) * gamma' + beta.
    Returns (y, h or None, mean or None, rstd or None). h_out=True allocates h
    (False skips it; a tensor, e.g. x itself, receives it); stats=True
    allocates the fp32 mean / rstd the backward needs (or pass the pair)."""
    T, H = _rows2d(x, "x")
    _need(residual, "residual", (T, H), _res_dtypes(x))
    _need(gamma, "gamma", (H,), (x.dtype,))
    _opt(beta, "beta", (H,), (x.dtype,))
    dev = _gpu(stream, ("x", x), ("residual", residual), ("gamma", gamma), ("beta", beta))
    if h_out is True:
        h_out = torch.empty_like(x)
    elif h_out is False or h_out is None:
        h_out = None
    else:
        _out(h_out, "h_out", (T, H), x.dtype, dev)
    y = _out(y, "y", (T, H), x.dtype, dev)
    mean = rstd = None
    if stats is True:
        mean = torch.empty(T, dtype=torch.float32, device=dev)
        rstd = torch.empty(T, dtype=torch.float32, device=dev)
    elif stats:
        mean, rstd = stats
        _grad_out(mean, "mean", T, dev)
        _grad_out(rstd, "rstd", T, dev)
    _check("mb_add_layer_norm_fwd", lib().mb_add_layer_norm_fwd(
        _p(x), _p(residual), _dt(residual), _p(gamma), _p(beta), float(eps), int(bool(zero_centered_gamma)),
        _p(h_out), _p(y), _p(mean), _p(rstd), T, H, _dt(x), _stream(dev, stream)))
    return y, h_out, mean, rstd


def mb_add_layer_norm_bwd_workspace(tokens, hidden, dtype, residual_dtype=None, with_param_grads=True) -> int:
    rdt = residual_dtype or dtype
    return int(lib().mb_add_layer_norm_bwd_workspace(tokens, hidden, DTYPES[dtype], DTYPES[rdt],
                                                     int(bool(with_param_grads))))


def mb_set_layer_norm_team_wait(polls: int) -> None:
    """Test-only: polls a block of the team-split LayerNorm backward makes for
    a partner's row sums before computing them itself (negative: the
    default). Outputs do not depend on it."""
    lib().mb_set_layer_norm_team_wait(int(polls))


def mb_add_layer_norm_bwd(dy, h, gamma, mean, rstd, zero_centered_gamma=False, dh_in=None, residual_dtype=None,
                          dx=None, dresidual=False, dgamma=True, dbeta=True, ws=None, stream=None):
    """Returns (dx, dresidual or None, dgamma or None, dbeta or None).
    residual_dtype (default: dh_in's dtype, else h's) is the dtype of dh_in and
    dresidual; dresidual=True allocates it."""
    T, H = _rows2d(h, "h")
    _need(dy, "dy", (T, H), (h.dtype,))
    _need(gamma, "gamma", (H,), (h.dtype,))
    _need(mean, "mean", (T,), (torch.float32,))
    _need(rstd, "rstd", (T,), (torch.float32,))
    rdt = residual_dtype or (dh_in.dtype if isinstance(dh_in, torch.Tensor) else h.dtype)
    if rdt not in _res_dtypes(h):
        raise ValueError(f"residual_dtype must be {h.dtype} or torch.float32, got {rdt}")
    _opt(dh_in, "dh_in", (T, H), (rdt,))
    dev = _gpu(stream, ("h", h), ("dy", dy), ("gamma", gamma), ("mean", mean), ("rstd", rstd),
               ("dh_in", dh_in))
    dx = _out(dx, "dx", (T, H), h.dtype, dev)
    if dresidual is True:
        dresidual = torch.empty((T, H), dtype=rdt, device=dev)
    elif dresidual is False or dresidual is None:
        dresidual = None
    else:
        _out(dresidual, "dresidual", (T, H), rdt, dev)
    dgamma = _grad_out(dgamma, "dgamma", H, dev)
    dbeta = _grad_out(dbeta, "dbeta", H, dev)
    ws, nws = _ws(ws, mb_add_layer_norm_bwd_workspace(T, H, h.dtype, rdt, dgamma is not None or dbeta is not None),
                  dev)
    _check("mb_add_layer_norm_bwd", lib().mb_add_layer_norm_bwd(
        _p(dy), _p(h), _p(gamma), _p(mean), _p(rstd), int(bool(zero_centered_gamma)), _p(dh_in), DTYPES[rdt],
        _p(dx), _p(dresidual), _p(dgamma), _p(dbeta), _p(ws), nws, T, H, _dt(h), _stream(dev, stream)))
    return dx, dresidual, dgamma, dbeta


# ------------------------------------------------------------------ weighted squared ReLU

def mb_weighted_squared_relu_fwd(x, weights=None, out=None, stream=None):
    """relu(x)^2 * weights[t] (weights None: the plain squared ReLU); out=x runs in place."""
    T, H = _rows2d(x, "x")
    _opt(weights, "weights", (T,), _FLOAT)
    dev = _gpu(stream, ("x", x), ("weights", weights))
    out = _out(out, "out", (T, H), x.dtype, dev)
    wdt = _dt(weights) if weights is not None else 0
    _check("mb_weighted_squared_relu_fwd", lib().mb_weighted_squared_relu_fwd(
        _p(x), _p(weights), wdt, _p(out), T, H, _dt(x), _stream(dev, stream)))
    return out


def mb_weighted_squared_relu_bwd_workspace(tokens, hidden, dtype, with_dweights=True) -> int:
    return int(lib().mb_weighted_squared_relu_bwd_workspace(tokens, hidden, DTYPES[dtype], int(bool(with_dweights))))


def mb_weighted_squared_relu_bwd(g, x, weights=None, dx=None, dweights=None, ws=None, stream=None):
    """Returns (dx, dweights or None); dweights defaults to True when weights are given."""
    T, H = _rows2d(x, "x")
    _need(g, "g", (T, H), (x.dtype,))
    _opt(weights, "weights", (T,), _FLOAT)
    dev = _gpu(stream, ("x", x), ("g", g), ("weights", weights))
    if dweights is None:
        dweights = weights is not None
    dx = _out(dx, "dx", (T, H), x.dtype, dev)
    dweights = _grad_out(dweights, "dweights", T, dev)
    ws, nws = _ws(ws, mb_weighted_squared_relu_bwd_workspace(T, H, x.dtype, dweights is not None), dev)
    wdt = _dt(weights) if weights is not None else 0
    _check("mb_weighted_squared_relu_bwd", lib().mb_weighted_squared_relu_bwd(
        _p(g), _p(x), _p(weights), wdt, _p(dx), _p(dweights), _p(ws), nws, T, H, _dt(x), _stream(dev, stream)))
    return dx, dweights
