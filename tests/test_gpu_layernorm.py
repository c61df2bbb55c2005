"""GPU parity of residual add + LayerNorm (forward and backward) against the
oracle, through the C ABI.

Shapes cover every row-group shape the kernels pick (4 rows of 64 threads per
block with 1, 2 or 4 vectors per thread; 256 and 1024 threads per row; rows
of 1025-2048 vectors, whose backward is a resident block per compute unit
walking a range of rows; the wide rows, whose backward is a row-sum kernel
and a column-strip kernel),
ragged rows (vectors that exist for only some threads), more rows than
blocks (grid-stride rows and more than 32 partial rows), and every dtype
pair. h is compared bit for bit; y, dx and dresidual within the derived
bound K * 2^-24 * mag (mag from the oracle: the size of the terms the fp32
evaluation combines; K = 128 covers the summation depth of the row sums, at
most 86 additions, plus the rounding of the normalisation); mean and rstd
within the same bound on their own scale; dgamma and dbeta as reductions.
"""
import numpy as np
import pytest
import torch

import oracle
import transformer_elementwise_epilogues_amd as mb
from transformer_elementwise_epilogues_amd import synthetic
from tolerances import assert_close_bounded, assert_reduction_close, to_storage as st, values as values_of

pytestmark = pytest.mark.gpu
DEV = "cuda"
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
U = 2.0**-24
K = 128.0

PAIRS = [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32"), ("f16", "f16"), ("f16", "f32")]


def hidden_cases(dt, rdt):
    """(T, H) per row-group shape, for elements-per-vector E."""
    E = 4 if (dt == "f32" or rdt == "f32") else 8
    # vectors per row; from 1025 to 2048 the backward is the resident block
    # walking a range of rows, beyond 2048 the wide-row pair (row sums, then
    # column strips walking the rows backwards), and the forward of 4096 runs
    # 512 threads of 8
    # (one vector per row: 4 bf16 beside an fp32 residual planned a column
    # strip of zero vectors for the unused parameter-gradient kernel, a host
    # division by zero that the sanitized build of the planner found)
    widths = [1, 3, 33, 128, 255, 512, 1021, 1536, 2048, 4096, 8192]
    rows = {1: 11, 3: 17, 33: 37, 128: 65, 255: 9, 512: 20, 1021: 6, 1536: 5, 2048: 300, 4096: 4, 8192: 3}
    return [(rows[w], w * E) for w in widths]


CASES = [(dt, rdt, T, H) for dt, rdt in PAIRS for (T, H) in hidden_cases(dt, rdt)]


def say(msg):
    print(f"[ln] {msg}", flush=True)


def inputs(dt, rdt, T, H, seed, scale=1.0, shift=0.0):
    x = synthetic.draw(seed, (T, H), "normal", scale, dt)
    r = synthetic.draw(seed + 1, (T, H), "normal", scale, rdt)
    if shift:
        x = (x.float() + shift).to(TD[dt])
    g = synthetic.draw(seed + 2, (H,), "normal", 0.3, dt)
    g = (g.float() + 1.0).to(TD[dt])
    b = synthetic.draw(seed + 3, (H,), "normal", 0.2, dt)
    return x, r, g, b


def check_fwd(dt, rdt, x, r, g, b, eps, zc, out, what):
    y, h, mean, rstd = out
    oh, oy, oy64, omag, omean, orstd = oracle.add_layer_norm_fwd(dt, st(x), st(r), rdt, st(g),
                                                                 None if b is None else st(b), eps, zc)
    assert np.array_equal(st(h), oh), f"{what}: h differs from the oracle's"
    s1 = assert_close_bounded(st(y), oy, oy64, K * U * omag, dt, f"{what} y")
    mean_abs = h.double().abs().mean(1).cpu().numpy()
    em = np.abs(mean.cpu().double().numpy() - omean)
    assert np.all(em <= K * U * mean_abs + 1e-30), f"{what} mean: worst {float(np.max(em / (K * U * mean_abs + 1e-30)))}"
    er = np.abs(rstd.cpu().double().numpy() - orstd) / orstd
    assert np.all(er <= K * U), f"{what} rstd: worst relative {float(er.max())}"
    return s1, oh


@pytest.mark.parametrize("dt,rdt,T,H", CASES)
def test_ln_fwd_bwd(dt, rdt, T, H):
    seed = 100 + H % 997
    x, r, g, b = inputs(dt, rdt, T, H, seed)
    out = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV), eps=1e-5)
    s1, oh = check_fwd(dt, rdt, x, r, g, b, 1e-5, False, out, f"fwd {dt}/{rdt} {T}x{H}")
    say(f"fwd {dt}/{rdt} {T}x{H}: {s1}")
    y, h, mean, rstd = out
    dy = synthetic.draw(seed + 4, (T, H), "normal", 1.0, dt).to(DEV)
    up = synthetic.draw(seed + 5, (T, H), "normal", 0.5, rdt).to(DEV)
    dx, dres, dgam, dbet = mb.mb_add_layer_norm_bwd(dy, h, g.to(DEV), mean, rstd, dh_in=up, dresidual=True)
    odx, odx64, omag, odres, odg, odb = oracle.add_layer_norm_bwd(dt, st(dy), oh, st(g), 1e-5, False,
                                                                  dh_in=st(up), res_dt=rdt)
    s2 = assert_close_bounded(st(dx), odx, odx64, K * U * omag, dt, f"bwd {dt}/{rdt} {T}x{H} dx")
    s3 = assert_close_bounded(st(dres), odres, odx64, K * U * omag, rdt, f"bwd {dt}/{rdt} {T}x{H} dres")
    say(f"bwd {dt}/{rdt} {T}x{H}: dx {s2} dres {s3}")
    say(f"dgamma {assert_reduction_close(dgam.cpu().numpy(), odg, 'dgamma')} "
        f"dbeta {assert_reduction_close(dbet.cpu().numpy(), odb, 'dbeta')}")


# The hidden sizes the page lists for the persistent LayerNorm kernel [fusions
# §5.3]: every one runs here, bf16 with an fp32 residual (its 8-byte pieces)
# and with a bf16 one, zero-centred gamma on alternate sizes.
PAGE_HIDDEN = [1024, 1536, 2048, 2304, 3072, 3840, 4096, 5120, 6144, 8192, 10240, 12288, 12800, 15360, 16384,
               18432, 20480, 24576, 25600, 30720, 32768, 40960, 49152, 65536]


@pytest.mark.parametrize("rdt", ["bf16", "f32"])
@pytest.mark.parametrize("H", PAGE_HIDDEN)
def test_ln_page_hidden_sizes(H, rdt):
    """Forward and backward (with dh_in, dresidual and both parameter
    gradients) at each listed hidden size over 300 rows against the oracle:
    h bit for bit, y, dx and dresidual within the derived bound, dgamma and
    dbeta to 1e-3 of the fp64 sums. Rows of 16-bit elements beside an fp32
    residual go up to 32768: the wider listed sizes must be refused
    (MB_ERR_SHAPE)."""
    dt = "bf16"
    T = 300
    if rdt == "f32" and H > 32768:
        x = torch.zeros(4, H, dtype=torch.bfloat16, device=DEV)
        r = torch.zeros(4, H, dtype=torch.float32, device=DEV)
        gm = torch.ones(H, dtype=torch.bfloat16, device=DEV)
        with pytest.raises(mb.MBError, match="MB_ERR_SHAPE"):
            mb.mb_add_layer_norm_fwd(x, r, gm)
        return
    zc = PAGE_HIDDEN.index(H) % 2 == 1
    seed = 700 + PAGE_HIDDEN.index(H)
    x, r, g, b = inputs(dt, rdt, T, H, seed)
    if zc:
        g = (g.float() - 1.0).to(TD[dt])  # zero-centred: the kernel applies gamma + 1
    out = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV), eps=1e-5, zero_centered_gamma=zc)
    s1, oh = check_fwd(dt, rdt, x, r, g, b, 1e-5, zc, out, f"page fwd {dt}/{rdt} {T}x{H}")
    y, h, mean, rstd = out
    dy = synthetic.draw(seed + 4, (T, H), "normal", 1.0, dt).to(DEV)
    up = synthetic.draw(seed + 5, (T, H), "normal", 0.5, rdt).to(DEV)
    dx, dres, dgam, dbet = mb.mb_add_layer_norm_bwd(dy, h, g.to(DEV), mean, rstd, zc, dh_in=up, dresidual=True)
    odx, odx64, omag, odres, odg, odb = oracle.add_layer_norm_bwd(dt, st(dy), oh, st(g), 1e-5, zc,
                                                                  dh_in=st(up), res_dt=rdt)
    s2 = assert_close_bounded(st(dx), odx, odx64, K * U * omag, dt, f"page bwd {dt}/{rdt} {T}x{H} dx")
    assert_close_bounded(st(dres), odres, odx64, K * U * omag, rdt, f"page bwd {dt}/{rdt} {T}x{H} dres")
    say(f"page {dt}/{rdt} {T}x{H} zc={zc}: fwd {s1} dx {s2}")
    assert_reduction_close(dgam.cpu().numpy(), odg, "dgamma")
    assert_reduction_close(dbet.cpu().numpy(), odb, "dbeta")


@pytest.mark.parametrize("dt,rdt", PAIRS)
@pytest.mark.parametrize("zc", [False, True])
@pytest.mark.parametrize("width", ["row", "block", "wide"])
def test_ln_options_beta_none_small_variance(dt, rdt, zc, width):
    # block: 2048 vectors, the resident-block backward; wide: 4096, the two-kernel one
    E = 4 if (dt == "f32" or rdt == "f32") else 8
    T, H = {"row": (40, 1024), "block": (12, 2048 * E), "wide": (12, 4096 * E)}[width]
    x, r, g, _ = inputs(dt, rdt, T, H, 7, scale=2e-3, shift=0.25)
    if zc:
        g = (g.float() - 1.0).to(TD[dt])  # zero-centred weights
    out = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), None, eps=1e-5, zero_centered_gamma=zc)
    s, oh = check_fwd(dt, rdt, x, r, g, None, 1e-5, zc, out, f"options {dt}/{rdt} zc={zc}")
    say(f"options {dt}/{rdt} zc={zc}: {s}")
    y, h, mean, rstd = out
    dy = synthetic.draw(8, (T, H), "normal", 1.0, dt).to(DEV)
    dx, _, dgam, dbet = mb.mb_add_layer_norm_bwd(dy, h, g.to(DEV), mean, rstd, zero_centered_gamma=zc,
                                                 residual_dtype=TD[rdt])
    odx, odx64, omag, _, odg, odb = oracle.add_layer_norm_bwd(dt, st(dy), oh, st(g), 1e-5, zc, res_dt=rdt,
                                                              want_dres=False)
    assert_close_bounded(st(dx), odx, odx64, K * U * omag, dt, f"options bwd {dt}/{rdt} zc={zc}")
    assert_reduction_close(dgam.cpu().numpy(), odg, "dgamma")
    assert_reduction_close(dbet.cpu().numpy(), odb, "dbeta")


def test_ln_many_rows_tall_partials():
    # 5000 rows of 1024 bf16: 4 rows per block, 512 blocks, 512 partial rows
    # (the chunked column sum), grid-stride rows
    dt = rdt = "bf16"
    T, H = 5000, 1024
    x, r, g, b = inputs(dt, rdt, T, H, 21)
    out = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV))
    s, oh = check_fwd(dt, rdt, x, r, g, b, 1e-5, False, out, "many rows")
    y, h, mean, rstd = out
    dy = synthetic.draw(22, (T, H), "normal", 1.0, dt).to(DEV)
    dx, _, dgam, dbet = mb.mb_add_layer_norm_bwd(dy, h, g.to(DEV), mean, rstd)
    odx, odx64, omag, _, odg, odb = oracle.add_layer_norm_bwd(dt, st(dy), oh, st(g), 1e-5, want_dres=False)
    assert_close_bounded(st(dx), odx, odx64, K * U * omag, dt, "many rows dx")
    say(f"many rows dgamma {assert_reduction_close(dgam.cpu().numpy(), odg, 'dgamma')}")
    assert_reduction_close(dbet.cpu().numpy(), odb, "dbeta")
    # bit-reproducible
    dx2, _, dgam2, dbet2 = mb.mb_add_layer_norm_bwd(dy, h, g.to(DEV), mean, rstd)
    assert torch.equal(dx.view(torch.int16), dx2.view(torch.int16))
    assert torch.equal(dgam.view(torch.int32), dgam2.view(torch.int32))
    assert torch.equal(dbet.view(torch.int32), dbet2.view(torch.int32))


@pytest.mark.parametrize("dt,rdt,T,H", [("bf16", "bf16", 1100, 16384), ("bf16", "bf16", 700, 12296),
                                         ("f16", "f32", 257, 8196), ("bf16", "bf16", 37, 65536)])
def test_ln_wide_backward_many_rows(dt, rdt, T, H):
    """The backward of rows over 1024 vectors over many rows: the resident
    blocks (2048 vectors, and 12296 bf16, 1537 vectors, ragged in a thread's
    last vector) walk several rows each; the wide-row pair (8196 beside an
    fp32 residual: 2049 vectors, the narrowest wide row, its last column
    strip ragged; and 8192 vectors) walks each row group from its last row
    down. dx, dresidual, dgamma and dbeta match the oracle and reproduce bit
    for bit."""
    say(f"wide bwd {dt}/{rdt} {T}x{H}")
    x, r, g, b = inputs(dt, rdt, T, H, 31)
    out = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV))
    _, oh = check_fwd(dt, rdt, x, r, g, b, 1e-5, False, out, "wide")
    y, h, mean, rstd = out
    dy = synthetic.draw(32, (T, H), "normal", 1.0, dt).to(DEV)
    up = synthetic.draw(33, (T, H), "normal", 1.0, rdt).to(DEV)
    dx, dres, dgam, dbet = mb.mb_add_layer_norm_bwd(dy, h, g.to(DEV), mean, rstd, dh_in=up, dresidual=True)
    odx, odx64, omag, odres, odg, odb = oracle.add_layer_norm_bwd(dt, st(dy), oh, st(g), 1e-5, False,
                                                                  dh_in=st(up), res_dt=rdt)
    assert_close_bounded(st(dx), odx, odx64, K * U * omag, dt, "wide dx")
    assert_close_bounded(st(dres), odres, odx64, K * U * omag, rdt, "wide dresidual")
    say(f"wide dgamma {assert_reduction_close(dgam.cpu().numpy(), odg, 'dgamma')}")
    assert_reduction_close(dbet.cpu().numpy(), odb, "dbeta")
    dx2, dres2, dgam2, dbet2 = mb.mb_add_layer_norm_bwd(dy, h, g.to(DEV), mean, rstd, dh_in=up, dresidual=True)
    for a, b2 in ((dx, dx2), (dres, dres2), (dgam, dgam2), (dbet, dbet2)):
        assert torch.equal(a.view(torch.uint8), b2.view(torch.uint8))


def test_ln_block_backward_flushes_column_sums():
    """Rows of 1025 vectors (8200 bf16: the last of a thread's four vectors
    exists for one thread only) over 16640 rows: on 256 compute units each
    resident block walks 65 rows, so it stores its dgamma / dbeta sums into
    its partial row after 64 rows and adds the last row's to them; the 65th
    row also reads its mean and rstd from the second chunk of the wave's
    statistics ring and runs as the odd row after the two-row loop. Every
    element of dx and dresidual, and both column sums, against the oracle
    (evaluated over row chunks, its column sums added in fp64); the result
    reproduces bit for bit."""
    dt = rdt = "bf16"
    T, H = 16640, 8200
    say(f"block bwd flush {dt}/{rdt} {T}x{H}")
    x, r, g, b = inputs(dt, rdt, T, H, 81)
    y, h, mean, rstd = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV))
    dy = synthetic.draw(82, (T, H), "normal", 1.0, dt)
    up = synthetic.draw(83, (T, H), "normal", 1.0, rdt)
    dx, dres, dgam, dbet = mb.mb_add_layer_norm_bwd(dy.to(DEV), h, g.to(DEV), mean, rstd, dh_in=up.to(DEV),
                                                    dresidual=True)
    again = mb.mb_add_layer_norm_bwd(dy.to(DEV), h, g.to(DEV), mean, rstd, dh_in=up.to(DEV), dresidual=True)
    for a, c in zip((dx, dres, dgam, dbet), again):
        assert torch.equal(a.view(torch.uint8), c.view(torch.uint8))
    hh, dx, dres = st(h), st(dx), st(dres)
    odg, odb = np.zeros(H), np.zeros(H)
    C = 2080
    for i in range(0, T, C):
        oh, *_ = oracle.add_layer_norm_fwd(dt, st(x[i:i + C]), st(r[i:i + C]), rdt, st(g), st(b), 1e-5, False)
        assert np.array_equal(hh[i:i + C], oh), f"h rows {i}.."
        odx, odx64, omag, odres, cg, cb = oracle.add_layer_norm_bwd(dt, st(dy[i:i + C]), oh, st(g), 1e-5, False,
                                                                    dh_in=st(up[i:i + C]), res_dt=rdt)
        assert_close_bounded(dx[i:i + C], odx, odx64, K * U * omag, dt, f"block dx rows {i}..")
        assert_close_bounded(dres[i:i + C], odres, odx64, K * U * omag, rdt, f"block dresidual rows {i}..")
        odg += cg
        odb += cb
    say(f"block dgamma {assert_reduction_close(dgam.cpu().numpy(), odg, 'dgamma')}")
    assert_reduction_close(dbet.cpu().numpy(), odb, "dbeta")


@pytest.mark.parametrize("dt,rdt,T,H", [("bf16", "bf16", 300, 32768), ("f16", "f32", 257, 8196),
                                         ("f32", "f32", 64, 32768), ("bf16", "bf16", 1100, 20480)])
def test_ln_team_backward_same_whether_partners_sums_arrive(dt, rdt, T, H):
    """Rows of 2049-8192 vectors split over a team of blocks (4, 3 of 683,
    8, and 3 of 854 vectors here, 1100 rows walking several per team): each
    block takes its partners' partial row sums from their published slots, or
    after its bounded wait computes them itself. With no wait at all every
    row goes the second way; dx, dresidual, dgamma and dbeta come out bit for
    bit the same, and match the oracle."""
    say(f"team bwd {dt}/{rdt} {T}x{H}")
    x, r, g, b = inputs(dt, rdt, T, H, 91)
    _, h, mean, rstd = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV))
    dy = synthetic.draw(92, (T, H), "normal", 1.0, dt).to(DEV)
    up = synthetic.draw(93, (T, H), "normal", 1.0, rdt).to(DEV)
    run = lambda: mb.mb_add_layer_norm_bwd(dy, h, g.to(DEV), mean, rstd, dh_in=up, dresidual=True)
    first = run()
    try:
        mb.mb_set_layer_norm_team_wait(0)
        alone = run()
    finally:
        mb.mb_set_layer_norm_team_wait(-1)
    for a, c in zip(first, alone):
        assert torch.equal(a.view(torch.uint8), c.view(torch.uint8))
    oh, *_ = oracle.add_layer_norm_fwd(dt, st(x), st(r), rdt, st(g), st(b), 1e-5, False)
    assert np.array_equal(st(h), oh)
    odx, odx64, omag, odres, odg, odb = oracle.add_layer_norm_bwd(dt, st(dy), oh, st(g), 1e-5, False,
                                                                  dh_in=st(up), res_dt=rdt)
    dx, dres, dgam, dbet = first
    assert_close_bounded(st(dx), odx, odx64, K * U * omag, dt, "team dx")
    assert_close_bounded(st(dres), odres, odx64, K * U * omag, rdt, "team dresidual")
    say(f"team dgamma {assert_reduction_close(dgam.cpu().numpy(), odg, 'dgamma')}")
    assert_reduction_close(dbet.cpu().numpy(), odb, "dbeta")


def test_ln_block_backward_long_walk_sampled_rows():
    """Rows of 1025 vectors (8200 bf16) over 130 rows per resident block (on
    256 compute units; more rows on fewer): each block reads its rows' mean
    and rstd from a two-chunk ring refilled every 64 rows, so rows 64, 128
    and 129 of a block read the second chunk, the first chunk refilled, and
    the second again. The oracle recomputes sampled rows one by one (each row's
    h, y, dx and dresidual depend on that row alone) from the same seeded
    inputs; every element of those rows within the derived bound."""
    dt = rdt = "bf16"
    H = 8200
    T = 256 * 130
    say(f"block bwd long walk {dt}/{rdt} {T}x{H}")
    gen = torch.Generator(device=DEV).manual_seed(4242)
    draw = lambda shape, sc: (torch.randn(shape, generator=gen, device=DEV) * sc).to(torch.bfloat16)
    x, r, dy, up = draw((T, H), 1.0), draw((T, H), 1.0), draw((T, H), 1.0), draw((T, H), 0.5)
    g = (draw((H,), 0.3).float() + 1.0).to(torch.bfloat16)
    b = draw((H,), 0.2)
    y, h, mean, rstd = mb.mb_add_layer_norm_fwd(x, r, g, b)
    dx, dres, _, _ = mb.mb_add_layer_norm_bwd(dy, h, g, mean, rstd, dh_in=up, dresidual=True)
    rpb = -(-T // min(T, torch.cuda.get_device_properties(0).multi_processor_count))
    rows = sorted({blk * rpb + o for blk in (0, 97, 255) for o in (0, 1, 63, 64, 65, 127, 128, 129)
                   if blk * rpb + o < T})
    idx = torch.tensor(rows, device=DEV)
    pick = lambda t: st(t.index_select(0, idx).cpu())
    oh, oy, oy64, omag, _, _ = oracle.add_layer_norm_fwd(dt, pick(x), pick(r), rdt, st(g.cpu()), st(b.cpu()),
                                                         1e-5, False)
    assert np.array_equal(pick(h), oh)
    assert_close_bounded(pick(y), oy, oy64, K * U * omag, dt, "long walk y")
    odx, odx64, bmag, odres, _, _ = oracle.add_layer_norm_bwd(dt, pick(dy), oh, st(g.cpu()), 1e-5, False,
                                                              dh_in=pick(up), res_dt=rdt)
    s1 = assert_close_bounded(pick(dx), odx, odx64, K * U * bmag, dt, "long walk dx")
    assert_close_bounded(pick(dres), odres, odx64, K * U * bmag, rdt, "long walk dresidual")
    say(f"long walk rows {rows[:4]}...: dx {s1}")


def test_ln_team_backward_beside_another_stream():
    """The team backward, its grid sized to the blocks the device holds at
    once, launched while a long streaming kernel on a second stream holds part
    of the device (either launch order): a block whose partners are not yet
    resident waits, within its bound, or leaves the row to the fix-up pass.
    With the default bound the partners arrive in time; with the wait cut to
    64 polls (test-only entry point) a third to a half of the rows took the
    fix-up pass when the other kernel went first (MI355X). Either way dx,
    dresidual, dgamma and dbeta come out bit for bit those of the call run
    alone."""
    dt = rdt = "bf16"
    T, H = 2048, 32768  # 4096 vectors: teams of 4
    say(f"team bwd beside a second stream {dt}/{rdt} {T}x{H}")
    x, r, g, b = inputs(dt, rdt, T, H, 95)
    gd = g.to(DEV)
    _, h, mean, rstd = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), gd, b.to(DEV))
    dy = synthetic.draw(96, (T, H), "normal", 1.0, dt).to(DEV)
    up = synthetic.draw(97, (T, H), "normal", 1.0, rdt).to(DEV)
    ref = mb.mb_add_layer_norm_bwd(dy, h, gd, mean, rstd, dh_in=up, dresidual=True)
    # a GeLU forward over 1 GiB in and out (a few hundred microseconds) on the other stream
    big = torch.full((16384, 32768), 0.5, dtype=torch.bfloat16, device=DEV)  # its values do not matter
    big_out = torch.empty_like(big)
    # outputs and workspace allocated up front, on the default stream
    outs = [tuple(torch.empty_like(t) for t in ref) for _ in range(4)]
    ws = torch.empty(mb.mb_add_layer_norm_bwd_workspace(T, H, h.dtype, up.dtype, True), dtype=torch.uint8,
                     device=DEV)
    torch.cuda.synchronize()
    s_ln, s_other = torch.cuda.Stream(), torch.cuda.Stream()
    for polls in (-1, 64):  # the default bound, then a short one
        mb.mb_set_layer_norm_team_wait(polls)
        try:
            for i, (dx, dres, dg, db) in enumerate(outs):
                for t in (dx, dres, dg, db):
                    t.fill_(float("nan"))
                torch.cuda.synchronize()
                ln = lambda: mb.mb_add_layer_norm_bwd(dy, h, gd, mean, rstd, dh_in=up, dx=dx, dresidual=dres,
                                                      dgamma=dg, dbeta=db, ws=ws, stream=s_ln)
                other = lambda: mb.mb_bias_gelu_fwd(big, None, out=big_out, stream=s_other)
                if i % 2 == 0:
                    other()
                    ln()
                else:
                    ln()
                    other()
                torch.cuda.synchronize()
                for a, c in zip(ref, (dx, dres, dg, db)):
                    assert torch.equal(a.view(torch.uint8), c.view(torch.uint8)), f"wait {polls}, launch {i}"
        finally:
            mb.mb_set_layer_norm_team_wait(-1)


@pytest.mark.parametrize("dt,rdt,T,H", [("bf16", "bf16", 520, 65536), ("f32", "f32", 300, 32768),
                                         ("bf16", "f32", 261, 32768)])
def test_ln_fwd_widest_rows_walk(dt, rdt, T, H):
    """The widest rows (8192 vectors) keep h in LDS and prefetch the next row:
    more rows than compute units, so blocks walk several rows (and the last
    ones fewer); every element against the oracle, bit-reproducible."""
    say(f"widest fwd {dt}/{rdt} {T}x{H}")
    x, r, g, b = inputs(dt, rdt, T, H, 71)
    out = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV), 1e-5, True)
    s1, _ = check_fwd(dt, rdt, x, r, g, b, 1e-5, True, out, f"widest {dt}/{rdt} {T}x{H}")
    say(f"widest fwd: {s1}")
    again = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV), 1e-5, True)
    for a, c in zip(out, again):
        assert torch.equal(a.view(torch.uint8), c.view(torch.uint8))
    # no stats and no h: the same y
    y2, h2, m2, s2 = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV), 1e-5, True, h_out=False,
                                              stats=False)
    assert h2 is None and m2 is None and torch.equal(y2.view(torch.uint8), out[0].view(torch.uint8))


@pytest.mark.parametrize("H", [1024, 16384, 24576])
def test_ln_in_place(H):
    """h over x and y over the residual; dx over dy and dresidual over dh_in.
    Up to 2048 vectors the in-place backward is the same kernel as the
    out-of-place one, bit for bit; wider rows split over a team of blocks
    out of place take the wide-row kernels in place (a team's fix-up pass
    rereads whole rows of dy, h and dh_in), so there the two are compared
    with the oracle."""
    dt = "bf16"
    T = 6
    x, r, g, b = inputs(dt, dt, T, H, 31)
    xd, rd, gd, bd = x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV)
    y_ref, h_ref, m_ref, s_ref = mb.mb_add_layer_norm_fwd(xd, rd, gd, bd)
    xi, ri = xd.clone(), rd.clone()
    y, h, m, s = mb.mb_add_layer_norm_fwd(xi, ri, gd, bd, h_out=xi, y=ri)  # h over x, y over the residual
    assert h.data_ptr() == xi.data_ptr() and y.data_ptr() == ri.data_ptr()
    assert torch.equal(xi.view(torch.int16), h_ref.view(torch.int16))
    assert torch.equal(ri.view(torch.int16), y_ref.view(torch.int16))
    dy = synthetic.draw(32, (T, H), "normal", 1.0, dt).to(DEV)
    up = synthetic.draw(33, (T, H), "normal", 1.0, dt).to(DEV)
    dx_ref, dr_ref, dg_ref, db_ref = mb.mb_add_layer_norm_bwd(dy, h_ref, gd, m_ref, s_ref, dh_in=up, dresidual=True)
    dyi, upi = dy.clone(), up.clone()
    dx, dr, dg, db = mb.mb_add_layer_norm_bwd(dyi, h_ref, gd, m_ref, s_ref, dh_in=upi, dx=dyi,
                                              dresidual=upi)  # dx over dy, dresidual over dh_in
    assert dx.data_ptr() == dyi.data_ptr() and dr.data_ptr() == upi.data_ptr()
    if H // 8 <= 2048:
        assert torch.equal(dyi.view(torch.int16), dx_ref.view(torch.int16))
        assert torch.equal(upi.view(torch.int16), dr_ref.view(torch.int16))
        assert torch.equal(dg.view(torch.int32), dg_ref.view(torch.int32))
        assert torch.equal(db.view(torch.int32), db_ref.view(torch.int32))
    oh, *_ = oracle.add_layer_norm_fwd(dt, st(x), st(r), dt, st(g), st(b), 1e-5, False)
    odx, odx64, omag, odres, odg, odb = oracle.add_layer_norm_bwd(dt, st(dy), oh, st(g), 1e-5, False,
                                                                  dh_in=st(up), res_dt=dt)
    for got in (dyi, dx_ref):
        assert_close_bounded(st(got), odx, odx64, K * U * omag, dt, f"in place dx {H}")
    for got in (upi, dr_ref):
        assert_close_bounded(st(got), odres, odx64, K * U * omag, dt, f"in place dresidual {H}")
    for got_g, got_b in ((dg, db), (dg_ref, db_ref)):
        assert_reduction_close(got_g.cpu().numpy(), odg, "in place dgamma")
        assert_reduction_close(got_b.cpu().numpy(), odb, "in place dbeta")


def test_ln_edge_cases():
    # a constant row (variance 0: rstd = 1/sqrt(eps), y = beta), one row, the
    # narrowest row, no stats, empty batches
    dt = "bf16"
    T, H = 3, 8
    x = torch.full((T, H), 1.5, dtype=torch.bfloat16)
    r = torch.zeros((T, H), dtype=torch.bfloat16)
    x[1] = torch.arange(H, dtype=torch.bfloat16)
    g = torch.ones(H, dtype=torch.bfloat16)
    b = torch.linspace(-1, 1, H).to(torch.bfloat16)
    out = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV))
    check_fwd(dt, dt, x, r, g, b, 1e-5, False, out, "edge")
    assert torch.equal(out[0][0].cpu().view(torch.int16), b.view(torch.int16))
    y2, h2, m2, s2 = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV), h_out=False, stats=False)
    assert h2 is None and m2 is None and torch.equal(y2.view(torch.int16), out[0].view(torch.int16))
    e = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
    ge = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    y0, h0, m0, s0 = mb.mb_add_layer_norm_fwd(e, e, ge)
    assert y0.shape == (0, 64)
    dx0, _, dg0, db0 = mb.mb_add_layer_norm_bwd(e, e, ge, m0, s0)
    torch.cuda.synchronize()
    assert dx0.shape == (0, 64) and torch.count_nonzero(dg0).item() == 0 and torch.count_nonzero(db0).item() == 0


@pytest.mark.parametrize("dt,rdt", [("bf16", "bf16"), ("bf16", "f32"), ("f32", "f32")])
@pytest.mark.parametrize("H", [1024, 16384, 32768])
def test_ln_non_finite_and_extreme_magnitude_rows(dt, rdt, H):
    """Rows holding a NaN, a +inf or a -inf (the whole row is NaN, as in the
    oracle: the mean is NaN or +-inf and the variance NaN), rows scaled to
    1e15 and to 1e-30 (the variance 1e30 and 1e-60, the latter far below eps),
    a row at 3 with a spread of 1e-3, and an ordinary row. The finite rows also go through the backward. Rows
    stay below 1e19: beyond it (x - mean)^2 overflows fp32 while the oracle's
    fp64 variance stays finite."""
    T = 7
    x, r, g, b = inputs(dt, rdt, T, H, 61)
    xf, rf = x.float(), r.float()
    xf[1, 17], xf[2, 300], xf[3, H - 1] = float("nan"), float("inf"), float("-inf")
    xf[4] *= 1e15
    rf[4] *= 1e15
    xf[5] *= 1e-30
    rf[5] *= 1e-30
    xf[6] = 3.0 + xf[6] * 1e-3  # a mean far from zero against the spread:
    rf[6] *= 1e-3  # the two-pass variance keeps it
    x, r = xf.to(TD[dt]), rf.to(TD[rdt])
    y, h, mean, rstd = mb.mb_add_layer_norm_fwd(x.to(DEV), r.to(DEV), g.to(DEV), b.to(DEV), eps=1e-5)
    oh, oy, oy64, omag, omean, orstd = oracle.add_layer_norm_fwd(dt, st(x), st(r), rdt, st(g), st(b), 1e-5, False)
    ky, kh = y.cpu().float().numpy(), h.cpu().float().numpy()
    bad = [1, 2, 3]
    for i in bad:
        assert np.isnan(ky[i]).all() and np.isnan(oy64[i]).all(), f"row {i}: y not all NaN"
        assert np.isnan(rstd[i].item()) and np.isnan(orstd[i]), f"row {i}: rstd"
        km, om = mean[i].item(), omean[i]
        assert (np.isnan(km) and np.isnan(om)) or km == om, f"row {i}: mean {km} vs {om}"
    hv = st(h)
    same = (hv == oh) | (np.isnan(kh) & np.isnan(values_of(oh, dt)))
    assert same.all(), "h differs from the oracle's"
    good = [0, 4, 5, 6]
    sel = np.array(good)
    s1 = assert_close_bounded(st(y)[sel], oy[sel], oy64[sel], (K * U * omag)[sel], dt, "extreme rows y")
    mean_abs = h.double().abs().mean(1).cpu().numpy()[sel]
    em = np.abs(mean.cpu().double().numpy()[sel] - omean[sel])
    assert np.all(em <= K * U * mean_abs + 1e-300), "extreme rows mean"
    er = np.abs(rstd.cpu().double().numpy()[sel] - orstd[sel]) / orstd[sel]
    assert np.all(er <= K * U), f"extreme rows rstd: worst relative {float(er.max())}"
    say(f"extreme rows {dt}/{rdt} fwd: {s1}")
    hg, mg, rg_ = h[sel].contiguous(), mean[sel].contiguous(), rstd[sel].contiguous()
    dy = synthetic.draw(62, (len(good), H), "normal", 1.0, dt).to(DEV)
    dx, _, dgam, dbet = mb.mb_add_layer_norm_bwd(dy, hg, g.to(DEV), mg, rg_, residual_dtype=TD[rdt])
    odx, odx64, omag2, _, odg, odb = oracle.add_layer_norm_bwd(dt, st(dy), oh[sel], st(g), 1e-5, False, res_dt=rdt,
                                                               want_dres=False)
    s2 = assert_close_bounded(st(dx), odx, odx64, K * U * omag2, dt, "extreme rows dx")
    assert_reduction_close(dgam.cpu().numpy(), odg, "extreme rows dgamma")
    assert_reduction_close(dbet.cpu().numpy(), odb, "extreme rows dbeta")
    say(f"extreme rows {dt}/{rdt} bwd: {s2}")


def test_ln_errors_on_device_tensors():
    x = torch.zeros((4, 60), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(60, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mb.MBError):
        mb.mb_add_layer_norm_fwd(x, x, g)  # 60 is not a multiple of 8
    x = torch.zeros((4, 64), dtype=torch.bfloat16, device=DEV)
    g = torch.ones(64, dtype=torch.bfloat16, device=DEV)
    with pytest.raises(mb.MBError):
        mb.mb_add_layer_norm_fwd(x, x, g, eps=-1.0)
    y, h, m, s = mb.mb_add_layer_norm_fwd(x, x, g)
    with pytest.raises(mb.MBError):
        mb.mb_add_layer_norm_bwd(x, h, g, m, s, ws=torch.zeros(4, dtype=torch.uint8, device=DEV))


@pytest.mark.parametrize("T,H", [(3000, 512), (40, 2048), (300, 16384), (300, 32768)])
def test_ln_bwd_each_param_gradient_alone_matches_both(T, H):
    """dgamma and dbeta share their column-sum launches when both are asked
    for; each alone comes out bit for bit the same (3000 rows: more than 32
    partial rows, the two-level sum; 16384: the resident-block kernel; 32768:
    the wide-row kernels), and dx does not depend on which parameter
    gradients are asked for."""
    dt = "bf16"
    x = synthetic.draw(501, (T, H), "normal", 1.0, dt).to(DEV)
    r = synthetic.draw(502, (T, H), "normal", 1.0, dt).to(DEV)
    g = synthetic.draw(503, (H,), "normal", 0.02, dt).to(DEV)
    b = synthetic.draw(504, (H,), "normal", 0.02, dt).to(DEV)
    dy = synthetic.draw(505, (T, H), "normal", 1.0, dt).to(DEV)
    _, h, mean, rstd = mb.mb_add_layer_norm_fwd(x, r, g, b)
    _, _, dg_both, dbt_both = mb.mb_add_layer_norm_bwd(dy, h, g, mean, rstd)
    _, _, dg_only, none_b = mb.mb_add_layer_norm_bwd(dy, h, g, mean, rstd, dbeta=False)
    _, _, none_g, dbt_only = mb.mb_add_layer_norm_bwd(dy, h, g, mean, rstd, dgamma=False)
    assert none_b is None and none_g is None
    assert torch.equal(dg_both.view(torch.int32), dg_only.view(torch.int32))
    assert torch.equal(dbt_both.view(torch.int32), dbt_only.view(torch.int32))
    dx_both, _, _, _ = mb.mb_add_layer_norm_bwd(dy, h, g, mean, rstd)
    dx_none, _, ng, nb = mb.mb_add_layer_norm_bwd(dy, h, g, mean, rstd, dgamma=False, dbeta=False)
    assert ng is None and nb is None
    assert torch.equal(dx_both.view(torch.int16), dx_none.view(torch.int16))
