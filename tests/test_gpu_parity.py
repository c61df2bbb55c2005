"""GPU parity of every entry point against the oracle, at sizes the oracle
finishes in about a second that still span several column strips, several
row groups and ragged tails in both directions, plus the edge cases.

All calls go through the C ABI (the ctypes binding passes device pointers).
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_elementwise_epilogues_amd as mb
from transformer_elementwise_epilogues_amd import synthetic
from tolerances import assert_close, assert_reduction_close, to_storage, values

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}


def gen(seed, shape, dt, sigma=1.0, dist="normal"):
    return synthetic.draw(seed, shape, dist, sigma, dt)


def st(t):
    return to_storage(t)


def log(name, stats):
    print(f"[parity] {name}: {stats}", flush=True)


# Shapes: (tokens, hidden) with hidden a multiple of the 16-byte vector. 1576
# bf16 = 197 vectors = 3 full strips + 5 lanes; 1028 fp32 = 257 vectors.
SHAPES = {"f32": [(777, 1028), (4, 8), (1, 4), (513, 64)],
          "bf16": [(1000, 1576), (4, 8), (3, 8), (1, 8), (257, 512)],
          "f16": [(999, 1576), (4, 8)]}
CASES = [(dt, s) for dt, ss in SHAPES.items() for s in ss]


# ------------------------------------------------------------------ GeLU

# exact=False: the tanh approximation; exact=True: the erf form.
GELU_FWD = {False: mb.mb_bias_gelu_fwd, True: mb.mb_bias_gelu_erf_fwd}
GELU_BWD = {False: mb.mb_bias_gelu_bwd, True: mb.mb_bias_gelu_erf_bwd}
EXACT = pytest.mark.parametrize("exact", [False, True], ids=["tanh", "erf"])


@EXACT
@pytest.mark.parametrize("dt,shape", CASES)
@pytest.mark.parametrize("with_bias", [True, False])
def test_gelu_fwd(dt, shape, with_bias, exact):
    T, H = shape
    y = gen(11, shape, dt, sigma=3.0)
    b = gen(12, (H,), dt, sigma=0.5) if with_bias else None
    out = GELU_FWD[exact](y.to(DEV), None if b is None else b.to(DEV))
    o, o64 = oracle.bias_gelu_fwd(dt, st(y), None if b is None else st(b), exact=exact)
    log(f"gelu_fwd exact={exact} {dt} {shape}", assert_close(st(out), o, o64, None, dt, "gelu fwd"))


@EXACT
@pytest.mark.parametrize("dt,shape", CASES)
def test_gelu_bwd(dt, shape, exact):
    T, H = shape
    y = gen(21, shape, dt, sigma=3.0)
    g = gen(22, shape, dt)
    b = gen(23, (H,), dt, sigma=0.5)
    dgrad, dbias = GELU_BWD[exact](g.to(DEV), y.to(DEV), b.to(DEV))
    d, d64, mag, db64 = oracle.bias_gelu_bwd(dt, st(g), st(y), st(b), exact=exact)
    log(f"gelu_bwd exact={exact} {dt} {shape}", assert_close(st(dgrad), d, d64, mag, dt, "gelu bwd dgrad"))
    log(f"gelu_dbias exact={exact} {dt} {shape}",
        assert_reduction_close(dbias.cpu().numpy(), db64, "gelu dbias"))


def test_gelu_erf_differs_from_tanh():
    # the two forms agree to about 1e-3 relative near |z| ~ 1-3 but not bit for
    # bit: a path that silently ran one for the other would be caught here
    y = gen(24, (64, 512), "f32", sigma=2.0).to(DEV)
    a = mb.mb_bias_gelu_fwd(y)
    e = mb.mb_bias_gelu_erf_fwd(y)
    diff = (a - e).abs().max().item()
    assert 1e-5 < diff < 1e-2


@EXACT
def test_gelu_bwd_dbias_optional_and_deterministic(exact):
    y = gen(31, (640, 2048), "bf16").to(DEV)
    g = gen(32, (640, 2048), "bf16").to(DEV)
    b = gen(33, (2048,), "bf16", 0.02).to(DEV)
    bwd = GELU_BWD[exact]
    d1, db1 = bwd(g, y, b)
    d2, db2 = bwd(g, y, b)
    d3, none = bwd(g, y, b, dbias=False)
    assert none is None
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    assert torch.equal(d1.view(torch.int16), d3.view(torch.int16))
    assert torch.equal(db1.view(torch.int32), db2.view(torch.int32))


@EXACT
def test_gelu_in_place(exact):
    y = gen(41, (300, 1024), "bf16").to(DEV)
    b = gen(42, (1024,), "bf16", 0.02).to(DEV)
    ref = GELU_FWD[exact](y, b)
    y2 = y.clone()
    GELU_FWD[exact](y2, b, out=y2)
    assert torch.equal(ref.view(torch.int16), y2.view(torch.int16))
    g = gen(43, (300, 1024), "bf16").to(DEV)
    d_ref, db_ref = GELU_BWD[exact](g, y, b)
    g2 = g.clone()
    d_in, db_in = GELU_BWD[exact](g2, y, b, dgrad=g2)
    assert d_in.data_ptr() == g2.data_ptr()
    assert torch.equal(d_ref.view(torch.int16), g2.view(torch.int16))
    assert torch.equal(db_ref.view(torch.int32), db_in.view(torch.int32))


@EXACT
def test_gelu_extreme_values(exact):
    vals = np.array([0.0, -0.0, 1e-30, -1e-30, 1e-8, -0.7525, -6.0, -8.0, -9.5, -10.0, -10.3, -10.7, -11.0,
                     -12.0, -20.0, 6.0, 12.0, 1e4, -1e4, 2e4, -2e4, 1e20, -1e20, 3e38, -3e38, np.nan], np.float32)
    H = 32
    y32 = np.resize(vals, (4, H)).astype(np.float32)
    g32 = np.linspace(-2, 2, 4 * H, dtype=np.float32).reshape(4, H)
    for dt in ("f32", "bf16", "f16"):
        y = torch.from_numpy(y32).to(TD[dt])
        g = torch.from_numpy(g32).to(TD[dt])
        out = GELU_FWD[exact](y.to(DEV))
        o, o64 = oracle.bias_gelu_fwd(dt, st(y), None, exact=exact)
        assert_close(st(out), o, o64, None, dt, f"gelu fwd extremes {dt}")
        dg, _ = GELU_BWD[exact](g.to(DEV), y.to(DEV), dbias=False)
        d, d64, mag, _ = oracle.bias_gelu_bwd(dt, st(g), st(y), None, exact=exact)
        assert_close(st(dg), d, d64, mag, dt, f"gelu bwd extremes {dt}")


@EXACT
def test_gelu_empty_tokens(exact):
    y = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    assert GELU_FWD[exact](y).shape == (0, 64)
    dg, db = GELU_BWD[exact](y, y, torch.zeros(64, dtype=torch.bfloat16, device=DEV))
    assert torch.count_nonzero(db).item() == 0 and db.shape == (64,)


# ------------------------------------------------------------------ dropout-add

BDA_TYPES = [("bf16", "f32"), ("bf16", "bf16"), ("f32", "f32"), ("f16", "f16"), ("f16", "f32")]


@pytest.mark.parametrize("dt,rdt", BDA_TYPES)
@pytest.mark.parametrize("p,offset", [(0.1, 0), (0.5, 7), (0.0, 0), (1.0, 0), (0.1, 2**33 + 5)])
def test_bda_train(dt, rdt, p, offset):
    T, H = (1000, 1576) if dt != "f32" else (777, 1028)
    x = gen(51, (T, H), dt)
    r = gen(52, (T, H), rdt)
    b = gen(53, (H,), dt, 0.02)
    seed = 1234
    out = mb.mb_bias_dropout_add_train(x.to(DEV), b.to(DEV), r.to(DEV), p, seed, offset)
    o, o64, mag = oracle.bias_dropout_add(dt, st(x), st(b), st(r), rdt, True, p, seed, offset)
    log(f"bda_train {dt}/{rdt} p={p}", assert_close(st(out), o, o64, mag, dt, "bda train"))
    bits = mb.mb_dropout_mask(T, H, p, seed, offset)
    assert np.array_equal(bits.cpu().numpy(), oracle.dropout_mask(T, H, p, seed, offset))


@pytest.mark.parametrize("dt,rdt", BDA_TYPES)
def test_bda_infer_and_in_place(dt, rdt):
    T, H = (1000, 1576) if dt != "f32" else (777, 1028)
    x = gen(61, (T, H), dt)
    r = gen(62, (T, H), rdt)
    b = gen(63, (H,), dt, 0.02)
    xd = x.to(DEV)
    out = mb.mb_bias_dropout_add_infer(xd, b.to(DEV), r.to(DEV))
    o, o64, mag = oracle.bias_dropout_add(dt, st(x), st(b), st(r), rdt, False)
    assert_close(st(out), o, o64, mag, dt, "bda infer")
    res = mb.mb_bias_dropout_add_infer(xd, b.to(DEV), r.to(DEV), out=xd)
    assert res.data_ptr() == xd.data_ptr()
    assert torch.equal(xd.cpu().view(torch.int16 if dt != "f32" else torch.int32),
                       out.cpu().view(torch.int16 if dt != "f32" else torch.int32))


def test_bda_p0_equals_infer_bitwise_and_p1_is_residual():
    T, H = 513, 2048
    x = gen(71, (T, H), "bf16").to(DEV)
    r = gen(72, (T, H), "f32").to(DEV)
    b = gen(73, (H,), "bf16", 0.02).to(DEV)
    a = mb.mb_bias_dropout_add_train(x, b, r, 0.0, 99)
    c = mb.mb_bias_dropout_add_infer(x, b, r)
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    one = mb.mb_bias_dropout_add_train(x, b, r, 1.0, 99)
    cast = r.to(torch.bfloat16)
    assert torch.equal(one.float(), cast.float())  # r' + 0 (-0 becomes +0, equal as values)


def test_bda_train_in_place_and_deterministic():
    T, H = 700, 4096
    x = gen(81, (T, H), "bf16").to(DEV)
    r = gen(82, (T, H), "bf16").to(DEV)
    b = gen(83, (H,), "bf16", 0.02).to(DEV)
    a = mb.mb_bias_dropout_add_train(x, b, r, 0.1, 5, 3)
    a2 = mb.mb_bias_dropout_add_train(x, b, r, 0.1, 5, 3)
    assert torch.equal(a.view(torch.int16), a2.view(torch.int16))
    r2 = r.clone()
    mb.mb_bias_dropout_add_train(x, b, r2, 0.1, 5, 3, out=r2)  # in place on the residual
    assert torch.equal(a.view(torch.int16), r2.view(torch.int16))


@pytest.mark.parametrize("T,H", [(1, 4), (3, 4), (5, 12), (37, 100), (1000, 1576)])
@pytest.mark.parametrize("p", [0.1, 0.5, 1 - 2.0**-24, 2.0**-32])
def test_mask_export_bit_exact(T, H, p):
    bits = mb.mb_dropout_mask(T, H, p, 2024, 11)
    assert np.array_equal(bits.cpu().numpy(), oracle.dropout_mask(T, H, p, 2024, 11))


def test_bda_dropped_nan_does_not_propagate():
    T, H, p, seed = 16, 64, 0.5, 3
    bits = np.unpackbits(oracle.dropout_mask(T, H, p, seed, 0), bitorder="little")[:T * H].reshape(T, H)
    x = gen(91, (T, H), "bf16")
    xn = x.clone()
    xn[torch.from_numpy(bits == 0)] = float("nan")
    r = gen(92, (T, H), "f32")
    out = mb.mb_bias_dropout_add_train(xn.to(DEV), None, r.to(DEV), p, seed)
    o, o64, mag = oracle.bias_dropout_add("bf16", st(xn), None, st(r), "f32", True, p, seed, 0)
    assert_close(st(out), o, o64, mag, "bf16", "bda nan")
    assert not torch.isnan(out).any()


# ------------------------------------------------------------------ gated units

GLU_CASES = [("swiglu", "bf16", None), ("swiglu", "bf16", "bf16"), ("swiglu", "bf16", "f32"),
             ("swiglu", "f32", "f32"), ("swiglu", "f16", "f16"), ("geglu", "bf16", None),
             ("geglu", "f32", None), ("geglu", "f16", None)]


def _glu_inputs(dt, wdt, T, H, seed, sigma=1.0):
    x = gen(seed, (T, 2 * H), dt, sigma)
    b = gen(seed + 1, (2 * H,), dt, 0.02)
    g = gen(seed + 2, (T, H), dt)
    w = gen(seed + 3, (T,), wdt, dist="uniform") if wdt else None
    return x, b, g, w


@pytest.mark.parametrize("act,dt,wdt", GLU_CASES)
@pytest.mark.parametrize("shape", [(600, 1576), (5, 8), (1, 16), (130, 512)])
def test_glu_fwd(act, dt, wdt, shape):
    T, H = shape
    if dt == "f32" and H % 4:
        pytest.skip("fp32 rows need H % 4 == 0")
    x, b, _, w = _glu_inputs(dt, wdt, T, H, 101, 2.0 if act == "geglu" else 1.0)
    if act == "swiglu":
        out = mb.mb_bias_swiglu_fwd(x.to(DEV), b.to(DEV), None if w is None else w.to(DEV))
    else:
        out = mb.mb_bias_geglu_fwd(x.to(DEV), b.to(DEV))
    o, o64 = oracle.bias_glu_fwd(act, dt, st(x), st(b), None if w is None else st(w), wdt)
    log(f"{act}_fwd {dt} w={wdt} {shape}", assert_close(st(out), o, o64, None, dt, f"{act} fwd"))


@pytest.mark.parametrize("act,dt,wdt", GLU_CASES)
@pytest.mark.parametrize("shape", [(600, 1576), (5, 8), (130, 512)])
def test_glu_bwd(act, dt, wdt, shape):
    T, H = shape
    x, b, g, w = _glu_inputs(dt, wdt, T, H, 201, 2.0 if act == "geglu" else 1.0)
    if act == "swiglu":
        din, dbias, dw = mb.mb_bias_swiglu_bwd(g.to(DEV), x.to(DEV), b.to(DEV), None if w is None else w.to(DEV))
    else:
        din, dbias = mb.mb_bias_geglu_bwd(g.to(DEV), x.to(DEV), b.to(DEV))
        dw = None
    d, d64, mag, db64, dw64 = oracle.bias_glu_bwd(act, dt, st(g), st(x), st(b), None if w is None else st(w), wdt)
    log(f"{act}_bwd {dt} w={wdt} {shape}", assert_close(st(din), d, d64, mag, dt, f"{act} bwd din"))
    log(f"{act}_dbias {dt}", assert_reduction_close(dbias.cpu().numpy(), db64, f"{act} dbias"))
    if w is not None:
        log(f"{act}_dweights {dt}", assert_reduction_close(dw.cpu().numpy(), dw64, f"{act} dweights"))


def test_glu_bwd_in_place_optional_outputs_and_deterministic():
    T, H = 333, 1024
    x, b, g, w = _glu_inputs("bf16", "bf16", T, H, 301)
    xd, bd, gd, wd = x.to(DEV), b.to(DEV), g.to(DEV), w.to(DEV)
    din1, db1, dw1 = mb.mb_bias_swiglu_bwd(gd, xd, bd, wd)
    din2, db2, dw2 = mb.mb_bias_swiglu_bwd(gd, xd, bd, wd)
    assert torch.equal(din1.view(torch.int16), din2.view(torch.int16))
    assert torch.equal(db1.view(torch.int32), db2.view(torch.int32))
    assert torch.equal(dw1.view(torch.int32), dw2.view(torch.int32))
    din3, none_b, none_w = mb.mb_bias_swiglu_bwd(gd, xd, bd, wd, dbias=False, dweights=False)
    assert none_b is None and none_w is None
    assert torch.equal(din1.view(torch.int16), din3.view(torch.int16))
    x2 = xd.clone()
    din4, db4, dw4 = mb.mb_bias_swiglu_bwd(gd, x2, bd, wd, din=x2)
    assert din4.data_ptr() == x2.data_ptr()
    assert torch.equal(din1.view(torch.int16), x2.view(torch.int16))
    assert torch.equal(db1.view(torch.int32), db4.view(torch.int32))


@pytest.mark.parametrize("act", ["swiglu", "wswiglu", "geglu"])
@pytest.mark.parametrize("dt,T,H", [("bf16", 600, 1576), ("f16", 5, 8), ("f32", 130, 512), ("bf16", 262150, 64)])
def test_glu_bwd_without_dbias(act, dt, T, H):
    """Without the bias gradient the gated backward takes its own launch shape
    (many short-lived blocks; at [262150, 64] the waves walk a second sweep of
    rows): din equals the oracle's and, bit for bit, that of the call that also
    sums dbias; the weights gradient (summed per row) is bit for bit the same."""
    x, _, g, w = _glu_inputs(dt, dt if act == "wswiglu" else None, T, H, 611)
    xd, gd = x.to(DEV), g.to(DEV)
    if act == "geglu":
        din, none_b = mb.mb_bias_geglu_bwd(gd, xd, None, dbias=False)
        din2, _ = mb.mb_bias_geglu_bwd(gd, xd, None)
        dw = dw2 = None
    else:
        wd = None if w is None else w.to(DEV)
        din, none_b, dw = mb.mb_bias_swiglu_bwd(gd, xd, None, wd, dbias=False, dweights=wd is not None)
        din2, _, dw2 = mb.mb_bias_swiglu_bwd(gd, xd, None, wd)
    assert none_b is None
    assert np.array_equal(st(din).view(np.uint8), st(din2).view(np.uint8))
    if dw is not None:
        assert torch.equal(dw.view(torch.int32), dw2.view(torch.int32))
    kind = "geglu" if act == "geglu" else "swiglu"
    d, d64, mag, _, dw64 = oracle.bias_glu_bwd(kind, dt, st(g), st(x), None, None if w is None else st(w), dt)
    log(f"{act}_bwd no dbias {dt} {T}x{H}", assert_close(st(din), d, d64, mag, dt, f"{act} bwd din, no dbias"))
    if dw is not None:
        assert_reduction_close(dw.cpu().numpy(), dw64, f"{act} dweights, no dbias")


def test_weighted_with_unit_weights_equals_unweighted():
    T, H = 257, 1536
    x, b, g, _ = _glu_inputs("bf16", None, T, H, 401)
    ones = torch.ones(T, dtype=torch.bfloat16, device=DEV)
    xd, bd, gd = x.to(DEV), b.to(DEV), g.to(DEV)
    a = mb.mb_bias_swiglu_fwd(xd, bd)
    c = mb.mb_bias_swiglu_fwd(xd, bd, ones)
    assert torch.equal(a.view(torch.int16), c.view(torch.int16))
    d1, db1, _ = mb.mb_bias_swiglu_bwd(gd, xd, bd)
    d2, db2, dw2 = mb.mb_bias_swiglu_bwd(gd, xd, bd, ones)
    assert torch.equal(d1.view(torch.int16), d2.view(torch.int16))
    assert torch.equal(db1.view(torch.int32), db2.view(torch.int32))


def test_glu_tail_inputs():
    # gate values deep in the negative tail, where gelu and its derivative are
    # tiny and the fp32 evaluation must stay out of the subnormal range
    T, H = 64, 256
    a = torch.linspace(-14, 4, T * H).reshape(T, H)
    up = gen(501, (T, H), "f32", 3.0)
    x = torch.cat([a, up], dim=1).to(torch.bfloat16)
    g = gen(502, (T, H), "bf16")
    for act in ("geglu", "swiglu"):
        if act == "geglu":
            out = mb.mb_bias_geglu_fwd(x.to(DEV))
            din, _ = mb.mb_bias_geglu_bwd(g.to(DEV), x.to(DEV), dbias=False)
        else:
            out = mb.mb_bias_swiglu_fwd(x.to(DEV))
            din, _, _ = mb.mb_bias_swiglu_bwd(g.to(DEV), x.to(DEV), dbias=False, dweights=False)
        o, o64 = oracle.bias_glu_fwd(act, "bf16", st(x), None)
        assert_close(st(out), o, o64, None, "bf16", f"{act} tail fwd")
        d, d64, mag, _, _ = oracle.bias_glu_bwd(act, "bf16", st(g), st(x), None)
        assert_close(st(din), d, d64, mag, "bf16", f"{act} tail bwd")


@pytest.mark.parametrize("dt", ["f32", "bf16", "f16"])
@pytest.mark.parametrize("weighted", [False, True])
def test_glu_extreme_values(dt, weighted):
    """Gate values at the infinities, NaN, huge finite values, the SiLU tail
    where sigma(a) is subnormal in fp32 (a < -87), the GeLU tail and the roots
    of both derivatives, against up values from tiny to huge (1e20), in both
    gated activations, forward and backward (NaN and inf follow the formulas).
    The deepest SiLU gate is -109: below |a| log2(e) = 158 the kernels flush
    the activation to zero, which is exact to tolerance only while the up
    value and gradient stay below about 2^16. Up values stay finite in each
    dtype (6e4 in fp16): an infinite one times an activation that is nonzero
    in fp64 but below fp32's range (gelu(-20) is about -1e-261) is inf in the
    fp64 oracle and 0 * inf = NaN in any fp32 evaluation. Weights are >= 1
    here: the kernels form products in fp32, and a weight below 1 would bring
    an intermediate that overflowed fp32 (silu(3e38) * 7) back into range in
    the fp64 oracle (zero and small weights are in the regular tests)."""
    gate = np.array([0.0, -0.0, 1e-30, -1e-30, -0.7525, -1.2785, -6.0, -10.3, -14.0, -20.0, -80.0, -87.0, -87.5,
                     -90.0, -95.0, -100.0, -104.0, -109.0, 3.0, 20.0, 90.0, 1e4, -1e4, 2e4, -2e4, 1e20, -1e20,
                     3e38, -3e38, np.inf, -np.inf, np.nan], np.float32)
    up = np.array([1.0, -2.5, 1e-3, 7.0, 6e4 if dt == "f16" else 1e20, -1e-20, 0.0, 300.0], np.float32)
    T, H = 8, 32
    a = np.stack([np.roll(gate, 3 * r) for r in range(T)])
    b = np.resize(up, (T, H))
    x32 = np.concatenate([a, b], axis=1)
    g32 = np.linspace(-2, 2, T * H, dtype=np.float32).reshape(T, H)
    x = torch.from_numpy(x32).to(TD[dt])
    g = torch.from_numpy(g32).to(TD[dt])
    w = torch.tensor([1.0, 1.5, 2.0, 3.0, 1.25, 4.0, 1.0, 2.5], dtype=TD[dt]) if weighted else None
    for act in ("swiglu", "geglu"):
        if act == "geglu" and weighted:
            continue
        if act == "swiglu":
            out = mb.mb_bias_swiglu_fwd(x.to(DEV), None, None if w is None else w.to(DEV))
            din, _, _ = mb.mb_bias_swiglu_bwd(g.to(DEV), x.to(DEV), None, None if w is None else w.to(DEV),
                                              dbias=False, dweights=False)
        else:
            out = mb.mb_bias_geglu_fwd(x.to(DEV))
            din, _ = mb.mb_bias_geglu_bwd(g.to(DEV), x.to(DEV), dbias=False)
        ws = None if w is None else st(w)
        o, o64 = oracle.bias_glu_fwd(act, dt, st(x), None, ws, dt if weighted else None)
        log(f"{act} extremes fwd {dt} w={weighted}", assert_close(st(out), o, o64, None, dt, f"{act} extremes fwd"))
        d, d64, mag, _, _ = oracle.bias_glu_bwd(act, dt, st(g), st(x), None, ws, dt if weighted else None)
        log(f"{act} extremes bwd {dt} w={weighted}", assert_close(st(din), d, d64, mag, dt, f"{act} extremes bwd"))


def test_glu_empty_tokens():
    x = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.empty((0, 32), dtype=torch.bfloat16, device=DEV)
    w = torch.empty((0,), dtype=torch.bfloat16, device=DEV)
    assert mb.mb_bias_swiglu_fwd(x, None, w).shape == (0, 32)
    din, db, dw = mb.mb_bias_swiglu_bwd(g, x, torch.zeros(64, dtype=torch.bfloat16, device=DEV), w)
    assert db.shape == (64,) and torch.count_nonzero(db).item() == 0 and dw.shape == (0,)


# ------------------------------------------------------------------ errors through the binding

def test_errors_on_device_tensors():
    y = torch.zeros((8, 24), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mb.MBError, match="MB_ERR_SHAPE"):
        mb.mb_bias_gelu_fwd(torch.zeros((8, 20), dtype=torch.bfloat16, device=DEV))
    flat = torch.zeros(8 * 24 + 1, dtype=torch.bfloat16, device=DEV)
    mis = flat[1:].view(8, 24)
    with pytest.raises(mb.MBError, match="MB_ERR_ALIGN"):
        mb.mb_bias_gelu_fwd(mis)
    with pytest.raises(mb.MBError, match="MB_ERR_PROB"):
        mb.mb_bias_dropout_add_train(y, None, y.clone(), 1.5, 1)
    x = torch.zeros((8, 48), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mb.MBError, match="MB_ERR_ALIAS"):
        mb.mb_bias_swiglu_fwd(x, out=x.view(-1)[:192].view(8, 24))  # output overlaps the input
    with pytest.raises(mb.MBError, match="MB_ERR_WORKSPACE"):
        mb.mb_bias_gelu_bwd(y, y, None, ws=torch.zeros(4, dtype=torch.uint8, device=DEV))


# ------------------------------------------------------------------ dropout-add backward

@pytest.mark.parametrize("dt,rdt", BDA_TYPES)
@pytest.mark.parametrize("p,offset", [(0.1, 0), (0.5, 7), (0.0, 0), (1.0, 0), (0.3, 2**33 + 5)])
def test_bda_bwd(dt, rdt, p, offset):
    T, H = (1000, 1576) if dt != "f32" else (777, 1028)
    g = gen(111, (T, H), dt)
    seed = 4321
    dx, dres, dbias = mb.mb_bias_dropout_add_bwd(g.to(DEV), p, seed, offset, residual_dtype=TD[rdt])
    odx, odx64, odres, odb = oracle.bias_dropout_add_bwd(dt, st(g), rdt, p, seed, offset)
    log(f"bda_bwd {dt}/{rdt} p={p}", assert_close(st(dx), odx, odx64, None, dt, "bda bwd dx"))
    assert np.array_equal(st(dres), odres), "dresidual must be g in the residual dtype, bit for bit"
    log(f"bda_bwd dbias {dt}", assert_reduction_close(dbias.cpu().numpy(), odb, "bda bwd dbias"))
    bits = np.unpackbits(mb.mb_dropout_mask(T, H, p, seed, offset).cpu().numpy(), bitorder="little")[:T * H]
    dropped = torch.from_numpy(bits.reshape(T, H) == 0)
    assert torch.count_nonzero(dx.cpu()[dropped]).item() == 0


@pytest.mark.parametrize("dt,rdt", BDA_TYPES)
@pytest.mark.parametrize("T,H", [(1000, 1576), (3, 8), (140001, 64)])
def test_bda_bwd_without_dbias(dt, rdt, T, H):
    """Without the bias gradient the backward takes its own launch shape (many
    short-lived blocks; at [140001, 64] the waves walk a second sweep of rows):
    dx and dresidual equal the oracle's and, bit for bit, those of the call
    that also sums dbias."""
    g = gen(131, (T, H), dt)
    p, seed, off = 0.1, 2468, 9
    gd = g.to(DEV)
    dx, dres, none = mb.mb_bias_dropout_add_bwd(gd, p, seed, off, residual_dtype=TD[rdt], dbias=False)
    assert none is None
    dx2, dres2, _ = mb.mb_bias_dropout_add_bwd(gd, p, seed, off, residual_dtype=TD[rdt])
    assert np.array_equal(st(dx).view(np.uint8), st(dx2).view(np.uint8))
    assert np.array_equal(st(dres).view(np.uint8), st(dres2).view(np.uint8))
    odx, odx64, odres, _ = oracle.bias_dropout_add_bwd(dt, st(g), rdt, p, seed, off)
    log(f"bda_bwd no dbias {dt}/{rdt} {T}x{H}", assert_close(st(dx), odx, odx64, None, dt, "bda bwd dx, no dbias"))
    assert np.array_equal(st(dres), odres)


def test_bda_bwd_matches_forward_mask_in_place_and_deterministic():
    T, H, p, seed, off = 640, 2048, 0.1, 99, 3
    x = gen(121, (T, H), "bf16").to(DEV)
    r = gen(122, (T, H), "f32").to(DEV)
    g = gen(123, (T, H), "bf16").to(DEV)
    out = mb.mb_bias_dropout_add_train(x, None, r, p, seed, off)
    dx, dres, db = mb.mb_bias_dropout_add_bwd(g, p, seed, off, residual_dtype=torch.float32)
    # the forward's keep decisions (mask export) decide where dx is g*s and where 0;
    # a dropped element of the forward is exactly the cast residual
    bits = np.unpackbits(mb.mb_dropout_mask(T, H, p, seed, off).cpu().numpy(), bitorder="little")[:T * H]
    keep = torch.from_numpy(bits.reshape(T, H) == 1).to(DEV)
    assert torch.count_nonzero(dx[~keep]).item() == 0
    assert torch.equal((dx[keep] != 0), (g[keep] != 0))
    assert torch.equal(out.float()[~keep], r.to(torch.bfloat16).float()[~keep])
    dx2, dres2, db2 = mb.mb_bias_dropout_add_bwd(g, p, seed, off, residual_dtype=torch.float32)
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(db.view(torch.int32), db2.view(torch.int32))
    g2 = g.clone()
    dx3, _, db3 = mb.mb_bias_dropout_add_bwd(g2, p, seed, off, residual_dtype=torch.float32, dx=g2, dresidual=False)
    assert dx3.data_ptr() == g2.data_ptr()
    assert torch.equal(dx.view(torch.int16), g2.view(torch.int16))
    assert torch.equal(db.view(torch.int32), db3.view(torch.int32))


def test_bda_bwd_empty_and_errors():
    g = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    dx, dres, db = mb.mb_bias_dropout_add_bwd(g, 0.1, 1)
    assert db.shape == (64,) and torch.count_nonzero(db).item() == 0
    g = torch.zeros((8, 64), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mb.MBError, match="MB_ERR_PROB"):
        mb.mb_bias_dropout_add_bwd(g, 1.5, 1)
    with pytest.raises(mb.MBError, match="MB_ERR_ALIAS"):
        mb.mb_bias_dropout_add_bwd(g, 0.1, 1, dx=g, dresidual=g)  # two outputs on one buffer


@pytest.mark.parametrize("shape", [(333, 1024), (4000, 64)])
def test_glu_bwd_each_reduction_alone_matches_both(shape):
    """dbias and dweights are summed in one launch when both are asked for and
    in a launch of their own otherwise; either way each comes out bit for bit
    the same (the (4000, 64) case has more than 32 partial rows of dbias)."""
    T, H = shape
    x, b, g, w = _glu_inputs("bf16", "f32", T, H, 311)
    xd, bd, gd, wd = x.to(DEV), b.to(DEV), g.to(DEV), w.to(DEV)
    _, db_both, dw_both = mb.mb_bias_swiglu_bwd(gd, xd, bd, wd, dbias=True, dweights=True)
    _, db_only, none_w = mb.mb_bias_swiglu_bwd(gd, xd, bd, wd, dbias=True, dweights=False)
    _, none_b, dw_only = mb.mb_bias_swiglu_bwd(gd, xd, bd, wd, dbias=False, dweights=True)
    assert none_w is None and none_b is None
    assert torch.equal(db_both.view(torch.int32), db_only.view(torch.int32))
    assert torch.equal(dw_both.view(torch.int32), dw_only.view(torch.int32))
    d, d64, mag, db64, dw64 = oracle.bias_glu_bwd("swiglu", "bf16", st(g), st(x), st(b), st(w), "f32")
    log("swiglu dbias (pair)", assert_reduction_close(db_both.cpu().numpy(), db64, "swiglu dbias"))
    log("swiglu dweights (pair)", assert_reduction_close(dw_both.cpu().numpy(), dw64, "swiglu dweights"))


@EXACT
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_gelu_every_half_precision_input(dt, exact):
    """Every finite bf16 / fp16 value as input (no bias), forward and backward
    with g = 1 and g = -3 against the oracle: the whole input space of the
    half-precision kernels, including the degree-5 erfc forward."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if dt == "bf16":
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
        keep = np.isfinite(vals)
        y = torch.from_numpy(vals[keep].copy()).to(torch.bfloat16)
    else:
        vals = bits.view(np.float16)
        keep = np.isfinite(vals)
        y = torch.from_numpy(vals[keep].copy())
    n = (y.numel() // 8) * 8
    y = y[:n].reshape(-1, 64 if n % 64 == 0 else 8)
    out = GELU_FWD[exact](y.to(DEV))
    o, o64 = oracle.bias_gelu_fwd(dt, st(y), None, exact=exact)
    log(f"gelu fwd every {dt} exact={exact}", assert_close(st(out), o, o64, None, dt, "gelu fwd every input"))
    for gval in (1.0, -3.0):
        g = torch.full_like(y, gval)
        dg, _ = GELU_BWD[exact](g.to(DEV), y.to(DEV), dbias=False)
        d, d64, mag, _ = oracle.bias_gelu_bwd(dt, st(g), st(y), None, exact=exact)
        log(f"gelu bwd every {dt} exact={exact} g={gval}", assert_close(st(dg), d, d64, mag, dt, "gelu bwd every input"))


@pytest.mark.parametrize("act", ["swiglu", "geglu"])
@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_glu_every_half_precision_gate(act, dt):
    """Every finite bf16 / fp16 value as the gate a (up half b = 0.75, no
    bias), forward and backward with g = -0.5 against the oracle (the up value
    and g keep every product finite in the output dtype)."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if dt == "bf16":
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
        keep = np.isfinite(vals)
        a = torch.from_numpy(vals[keep].copy()).to(torch.bfloat16)
    else:
        vals = bits.view(np.float16)
        keep = np.isfinite(vals)
        a = torch.from_numpy(vals[keep].copy())
    H = 64
    n = (a.numel() // H) * H
    a = a[:n].reshape(-1, H)
    x = torch.cat([a, torch.full_like(a, 0.75)], dim=1).contiguous()
    g = torch.full_like(a, -0.5)
    if act == "swiglu":
        out = mb.mb_bias_swiglu_fwd(x.to(DEV))
        din, _, _ = mb.mb_bias_swiglu_bwd(g.to(DEV), x.to(DEV), dbias=False)
    else:
        out = mb.mb_bias_geglu_fwd(x.to(DEV))
        din, _ = mb.mb_bias_geglu_bwd(g.to(DEV), x.to(DEV), dbias=False)
    o, o64 = oracle.bias_glu_fwd(act, dt, st(x), None, None, None)
    log(f"{act} fwd every {dt} gate", assert_close(st(out), o, o64, None, dt, f"{act} fwd every gate"))
    d, d64, mag, _, _ = oracle.bias_glu_bwd(act, dt, st(g), st(x), None, None, None)
    log(f"{act} bwd every {dt} gate", assert_close(st(din), d, d64, mag, dt, f"{act} bwd every gate"))


@pytest.mark.parametrize("dt", ["bf16", "f16"])
def test_bda_every_half_precision_input(dt):
    """Every finite bf16 / fp16 value as x, with a residual of 0.25 and a
    bias of -0.5, through the training (p = 0.1) and inference passes and
    the backward (g = x), against the oracle."""
    bits = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16)
    if dt == "bf16":
        vals = (bits.astype(np.uint32) << 16).view(np.float32)
        keep = np.isfinite(vals)
        x = torch.from_numpy(vals[keep].copy()).to(torch.bfloat16)
    else:
        vals = bits.view(np.float16)
        keep = np.isfinite(vals)
        x = torch.from_numpy(vals[keep].copy())
    H = 64
    n = (x.numel() // H) * H
    x = x[:n].reshape(-1, H)
    r = torch.full_like(x, 0.25)
    b = torch.full((H,), -0.5, dtype=x.dtype)
    p, seed, off = 0.1, 77, 3
    out = mb.mb_bias_dropout_add_train(x.to(DEV), b.to(DEV), r.to(DEV), p, seed, off)
    o, o64, mag = oracle.bias_dropout_add(dt, st(x), st(b), st(r), dt, True, p, seed, off)
    log(f"bda train every {dt}", assert_close(st(out), o, o64, mag, dt, "bda train every input"))
    inf_out = mb.mb_bias_dropout_add_infer(x.to(DEV), b.to(DEV), r.to(DEV))
    o, o64, mag = oracle.bias_dropout_add(dt, st(x), st(b), st(r), dt, False)
    log(f"bda infer every {dt}", assert_close(st(inf_out), o, o64, mag, dt, "bda infer every input"))
    dx, dres, _ = mb.mb_bias_dropout_add_bwd(x.to(DEV), p, seed, off, dbias=False)
    odx, odx64, odres, _ = oracle.bias_dropout_add_bwd(dt, st(x), dt, p, seed, off)
    log(f"bda bwd every {dt}", assert_close(st(dx), odx, odx64, None, dt, "bda bwd every input"))
    assert np.array_equal(st(dres), odres)


@EXACT
@pytest.mark.parametrize("T", [132, 2048, 2052])
def test_gelu_bwd_dbias_across_column_sum_paths(T, exact):
    """H = 16384 bf16 (32 column strips): T = 132 gives 33 partial rows (the
    one-launch fold of 2 chunks), 2048 gives 512 (16 chunks, the most one
    launch folds), 2052 gives 513 (17 chunks: the two-launch path). dbias on
    sampled columns against the oracle's fp64 sum over every row, and dgrad on
    sampled rows."""
    H = 16384
    y = gen(601, (T, H), "bf16", sigma=2.0)
    g = gen(602, (T, H), "bf16")
    b = gen(603, (H,), "bf16", sigma=0.5)
    dgrad, dbias = GELU_BWD[exact](g.to(DEV), y.to(DEV), b.to(DEV))
    cols = np.unique(np.concatenate([np.random.default_rng(T).choice(H, 256, replace=False), [0, H - 1]]))
    _, _, _, db64 = oracle.bias_gelu_bwd("bf16", st(g[:, cols]), st(y[:, cols]), st(b[cols]), exact=exact)
    log(f"gelu dbias T={T} exact={exact}", assert_reduction_close(dbias.cpu().numpy()[cols], db64, "gelu dbias"))
    rows = np.unique(np.concatenate([np.random.default_rng(T + 1).choice(T, 16, replace=False), [0, T - 1]]))
    d, d64, mag, _ = oracle.bias_gelu_bwd("bf16", st(g[rows]), st(y[rows]), st(b), exact=exact)
    log(f"gelu dgrad rows T={T}", assert_close(st(dgrad.cpu()[rows]), d, d64, mag, "bf16", "gelu dgrad rows"))
