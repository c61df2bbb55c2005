"""Seeded synthetic inputs for the fused epilogues (shared by tests and bench).

This module only draws random numbers and casts them to the storage dtype; it
holds none of the epilogues' arithmetic. Tensor ``k`` of workload ``c`` is
drawn from ``numpy.random.default_rng([1000 * c + k, chunk])`` in chunks of
2^22 elements (so several threads can draw one tensor and the result does
not depend on the thread count), as float32 ``standard_normal() * sigma`` or
``random()`` (uniform on [0, 1)), then cast to the storage dtype by
``torch.Tensor.to`` (round to nearest even). ``N(0, s)`` names the standard
deviation ``s``.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field

import numpy as np
import torch

CHUNK = 1 << 22
_DT = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def _workers() -> int:
    return max(1, min(16, os.cpu_count() or 1))


def draw(seed: int, shape, dist: str = "normal", sigma: float = 1.0, dtype: str = "bf16") -> torch.Tensor:
    """One seeded tensor on the CPU, in storage dtype ``dtype``."""
    n = int(np.prod(shape)) if len(shape) else 1
    out = torch.empty(n, dtype=_DT[dtype])
    nchunks = (n + CHUNK - 1) // CHUNK

    def fill(c):
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        g = np.random.default_rng([seed, c])
        if dist == "normal":
            v = g.standard_normal(hi - lo, dtype=np.float32)
            if sigma != 1.0:
                v *= np.float32(sigma)
        elif dist == "uniform":
            v = g.random(hi - lo, dtype=np.float32)
        else:
            raise ValueError(dist)
        out[lo:hi] = torch.from_numpy(v).to(out.dtype)

    if nchunks <= 1:
        for c in range(nchunks):
            fill(c)
    else:
        with ThreadPoolExecutor(_workers()) as ex:
            list(ex.map(fill, range(nchunks)))
    return out.reshape(tuple(shape))


@dataclass
class Tensor:
    k: int
    shape: tuple
    dtype: str
    dist: str = "normal"
    sigma: float = 1.0


@dataclass
class Workload:
    """A named workload: tensor recipes plus the op parameters."""
    c: int
    name: str
    tensors: dict
    params: dict = field(default_factory=dict)

    def tensor(self, name: str) -> torch.Tensor:
        t = self.tensors[name]
        return draw(1000 * self.c + t.k, t.shape, t.dist, t.sigma, t.dtype)


def _w(c, name, tensors, **params):
    return Workload(c, name, tensors, params)


WORKLOADS = {
    "gelu_f32_512x4096": _w(1, "gelu_f32_512x4096", {
        "y": Tensor(0, (512, 4096), "f32"),
        "bias": Tensor(1, (4096,), "f32", sigma=0.02),
        "g": Tensor(2, (512, 4096), "f32"),
    }),
    "bda_bf16_8192x4096_res_f32": _w(2, "bda_bf16_8192x4096_res_f32", {
        "x": Tensor(0, (8192, 4096), "bf16"),
        "bias": Tensor(1, (4096,), "bf16", sigma=0.02),
        "residual": Tensor(2, (8192, 4096), "f32"),
        "g": Tensor(3, (8192, 4096), "bf16"),  # upstream gradient for the backward
    }, p=0.1, seed=1234, offset=0),
    "swiglu_bf16_8192x14336": _w(3, "swiglu_bf16_8192x14336", {
        "in": Tensor(0, (8192, 28672), "bf16"),
        "bias": Tensor(1, (28672,), "bf16", sigma=0.02),
        "g": Tensor(2, (8192, 14336), "bf16"),
        "weights": Tensor(3, (8192,), "bf16", dist="uniform"),
    }),
    "geglu_bf16_16384x8192": _w(4, "geglu_bf16_16384x8192", {
        "in": Tensor(0, (16384, 16384), "bf16", sigma=2.0),
        "bias": Tensor(1, (16384,), "bf16", sigma=0.02),
        "g": Tensor(2, (16384, 8192), "bf16"),
    }),
    "layer_chain_bf16_t16384_h8192_f32768": _w(5, "layer_chain_bf16_t16384_h8192_f32768", {
        "attn_x": Tensor(0, (16384, 8192), "bf16"),
        "attn_residual": Tensor(1, (16384, 8192), "bf16"),
        "attn_bias": Tensor(2, (8192,), "bf16", sigma=0.02),
        "gelu_y": Tensor(3, (16384, 32768), "bf16"),
        "gelu_bias": Tensor(4, (32768,), "bf16", sigma=0.02),
        "gelu_g": Tensor(5, (16384, 32768), "bf16"),
        "mlp_x": Tensor(6, (16384, 8192), "bf16"),
        "mlp_residual": Tensor(7, (16384, 8192), "bf16"),
        "mlp_bias": Tensor(8, (8192,), "bf16", sigma=0.02),
        "attn_g": Tensor(9, (16384, 8192), "bf16"),  # upstream gradients of the two dropout-adds
        "mlp_g": Tensor(10, (16384, 8192), "bf16"),
    }, p=0.1, attn_seed=5001, mlp_seed=5002, offset=0),
    # residual add + LayerNorm after a layer's residual path, at the chain's
    # hidden size (8192 is on the persistent-kernel list); zero-centred gamma
    "add_ln_bf16_16384x8192": _w(6, "add_ln_bf16_16384x8192", {
        "x": Tensor(0, (16384, 8192), "bf16"),
        "residual": Tensor(1, (16384, 8192), "bf16"),
        "gamma": Tensor(2, (8192,), "bf16", sigma=0.02),
        "beta": Tensor(3, (8192,), "bf16", sigma=0.02),
        "dy": Tensor(4, (16384, 8192), "bf16"),
        "dh_in": Tensor(5, (16384, 8192), "bf16"),
    }, eps=1e-5, zero_centered_gamma=True),
    # MoE expert activation: weighted squared ReLU of the first expert GEMM's
    # output, per-token routing weights in fp32
    "wsrelu_bf16_8192x14336": _w(7, "wsrelu_bf16_8192x14336", {
        "x": Tensor(0, (8192, 14336), "bf16"),
        "g": Tensor(1, (8192, 14336), "bf16"),
        "weights": Tensor(2, (8192,), "f32", dist="uniform"),
    }),
    # the same at the widest hidden sizes of the persistent-kernel list
    "add_ln_bf16_8192x16384": _w(8, "add_ln_bf16_8192x16384", {
        "x": Tensor(0, (8192, 16384), "bf16"),
        "residual": Tensor(1, (8192, 16384), "bf16"),
        "gamma": Tensor(2, (16384,), "bf16", sigma=0.02),
        "beta": Tensor(3, (16384,), "bf16", sigma=0.02),
        "dy": Tensor(4, (8192, 16384), "bf16"),
        "dh_in": Tensor(5, (8192, 16384), "bf16"),
    }, eps=1e-5, zero_centered_gamma=True),
    "add_ln_bf16_2048x65536": _w(9, "add_ln_bf16_2048x65536", {
        "x": Tensor(0, (2048, 65536), "bf16"),
        "residual": Tensor(1, (2048, 65536), "bf16"),
        "gamma": Tensor(2, (65536,), "bf16", sigma=0.02),
        "beta": Tensor(3, (65536,), "bf16", sigma=0.02),
        "dy": Tensor(4, (2048, 65536), "bf16"),
        "dh_in": Tensor(5, (2048, 65536), "bf16"),
    }, eps=1e-5, zero_centered_gamma=True),
}
