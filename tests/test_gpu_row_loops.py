"""The row loops of the tiled kernels when a wave owns many rows: tall, narrow
inputs (one column strip, so every row group of the grid is a slice of one
16-byte column) make each wave walk several rows, run the software-pipelined
steady state (next rows' loads issued before this rows' arithmetic) and end in
the remainder loop, with a row count that is not a multiple of the rows in
flight. The smaller parity cases give each wave one or two rows.

Row counts per kernel, with the launch shapes of the library (blocks of 256
threads; G row groups; a wave's rows are S = 4 G apart):
- GeLU backward, 32768 blocks, 4 rows in flight: S = 131072, T = 5 S + r;
- gated backward, 512 blocks, 1 row in flight: S = 2048, T = 9 S + r;
- dropout-add backward, same dtype: 768 blocks, 2 bands: S = 3072;
  fp32 residual: 512 blocks, 2 rows in flight: S = 2048;
- dropout-add forward with an fp32 residual: 512 blocks, 2 in flight;
- squared-ReLU backward, 16384 blocks: S = 65536;
- forward kernels, 65536 blocks: S = 262144.
Any shape is valid input; these only decide how much of the loops runs.
Every output element is compared with the oracle, and the reductions over all
rows with the oracle's fp64 sums.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_elementwise_epilogues_amd as mb
from transformer_elementwise_epilogues_amd import synthetic
from tolerances import assert_close, assert_reduction_close, to_storage as st

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def gen(seed, shape, dt, sigma=1.0, dist="normal"):
    return synthetic.draw(seed, shape, dist, sigma, dt)


def log(name, stats):
    print(f"[row loops] {name}: {stats}", flush=True)


@pytest.mark.parametrize("exact", [False, True], ids=["tanh", "erf"])
@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_gelu_many_rows_per_wave(dt, exact):
    T, H = 5 * 131072 + 12345, 8
    y = gen(301, (T, H), dt, sigma=3.0)
    g = gen(302, (T, H), dt)
    b = gen(303, (H,), dt, sigma=0.5)
    fwd = mb.mb_bias_gelu_erf_fwd if exact else mb.mb_bias_gelu_fwd
    bwd = mb.mb_bias_gelu_erf_bwd if exact else mb.mb_bias_gelu_bwd
    out = fwd(y.to(DEV), b.to(DEV))
    dgrad, dbias = bwd(g.to(DEV), y.to(DEV), b.to(DEV))
    o, o64 = oracle.bias_gelu_fwd(dt, st(y), st(b), exact=exact)
    log(f"gelu fwd {dt} exact={exact} {T}x{H}", assert_close(st(out), o, o64, None, dt, "gelu fwd"))
    d, d64, mag, db64 = oracle.bias_gelu_bwd(dt, st(g), st(y), st(b), exact=exact)
    log(f"gelu bwd {dt} exact={exact} {T}x{H}", assert_close(st(dgrad), d, d64, mag, dt, "gelu bwd"))
    log(f"gelu dbias {dt}", assert_reduction_close(dbias.cpu().numpy(), db64, "gelu dbias"))


@pytest.mark.parametrize("act,wdt", [("swiglu", "bf16"), ("swiglu", None), ("geglu", None)])
def test_glu_bwd_many_rows_per_wave(act, wdt):
    dt = "bf16"
    T, H = 9 * 2048 + 1500, 8
    x = gen(311, (T, 2 * H), dt, 2.0 if act == "geglu" else 1.0)
    b = gen(312, (2 * H,), dt, 0.02)
    g = gen(313, (T, H), dt)
    w = gen(314, (T,), wdt, dist="uniform") if wdt else None
    if act == "swiglu":
        din, dbias, dw = mb.mb_bias_swiglu_bwd(g.to(DEV), x.to(DEV), b.to(DEV), None if w is None else w.to(DEV))
    else:
        din, dbias = mb.mb_bias_geglu_bwd(g.to(DEV), x.to(DEV), b.to(DEV))
        dw = None
    d, d64, mag, db64, dw64 = oracle.bias_glu_bwd(act, dt, st(g), st(x), st(b), None if w is None else st(w), wdt)
    log(f"{act} bwd w={wdt} {T}x{H}", assert_close(st(din), d, d64, mag, dt, f"{act} bwd din"))
    log(f"{act} dbias", assert_reduction_close(dbias.cpu().numpy(), db64, f"{act} dbias"))
    if w is not None:
        log(f"{act} dweights", assert_reduction_close(dw.cpu().numpy(), dw64, f"{act} dweights"))


@pytest.mark.parametrize("rdt,T", [("bf16", 2 * 3072 * 5 + 1001), ("f32", 2 * 2048 * 5 + 777)])
def test_bda_many_rows_per_wave(rdt, T):
    dt, H, p, seed, off = "bf16", 8, 0.1, 2024, 5
    x = gen(321, (T, H), dt)
    b = gen(322, (H,), dt, 0.02)
    r = gen(323, (T, H), rdt)
    out = mb.mb_bias_dropout_add_train(x.to(DEV), b.to(DEV), r.to(DEV), p, seed, off)
    o, o64, mag = oracle.bias_dropout_add(dt, st(x), st(b), st(r), rdt, True, p, seed, off)
    log(f"bda train {dt}/{rdt} {T}x{H}", assert_close(st(out), o, o64, mag, dt, "bda train"))
    g = gen(324, (T, H), dt)
    dx, dres, dbias = mb.mb_bias_dropout_add_bwd(g.to(DEV), p, seed, off, residual_dtype=TD[rdt])
    odx, odx64, odres, odb = oracle.bias_dropout_add_bwd(dt, st(g), rdt, p, seed, off)
    log(f"bda bwd {dt}/{rdt} {T}x{H}", assert_close(st(dx), odx, odx64, None, dt, "bda bwd dx"))
    assert np.array_equal(st(dres), odres), "dresidual must be g in the residual dtype, bit for bit"
    log(f"bda bwd dbias {rdt}", assert_reduction_close(dbias.cpu().numpy(), odb, "bda bwd dbias"))


def test_squared_relu_many_rows_per_wave():
    dt, wdt = "bf16", "f32"
    T, H = 3 * 65536 + 77, 8
    x = gen(331, (T, H), dt, 2.0)
    w = gen(332, (T,), wdt, dist="uniform")
    g = gen(333, (T, H), dt)
    out = mb.mb_weighted_squared_relu_fwd(x.to(DEV), w.to(DEV))
    o, o64 = oracle.weighted_squared_relu_fwd(dt, st(x), st(w), wdt)
    log(f"srelu fwd {T}x{H}", assert_close(st(out), o, o64, None, dt, "srelu fwd"))
    dx, dw = mb.mb_weighted_squared_relu_bwd(g.to(DEV), x.to(DEV), w.to(DEV))
    d, d64, odw = oracle.weighted_squared_relu_bwd(dt, st(g), st(x), st(w), wdt)
    log(f"srelu bwd {T}x{H}", assert_close(st(dx), d, d64, None, dt, "srelu bwd"))
    log("srelu dweights", assert_reduction_close(dw.cpu().numpy(), odw, "srelu dweights"))
