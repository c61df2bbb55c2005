"""The entry points under HIP graph capture: a captured sequence of fused ops
(dropout-add forward and backward, GeLU backward with its bias gradient,
weighted SwiGLU backward, residual add + LayerNorm forward and backward,
weighted squared ReLU backward) is replayed several times, with the
program's own eager work and synchronisations between the replays, and every
replay must equal the eager results bit for bit. The library issues only
kernel launches (no memsets, no allocations, no synchronisation), so it is
capturable as is."""
import pytest
import torch

import transformer_elementwise_epilogues_amd as mb
from transformer_elementwise_epilogues_amd import synthetic

pytestmark = pytest.mark.gpu
DEV = "cuda"


def bits(t):
    return t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)


def test_capture_and_replay_matches_eager():
    T, H = 1024, 2048
    x = synthetic.draw(1, (T, H), "normal", 1.0, "bf16").to(DEV)
    r = synthetic.draw(2, (T, H), "normal", 1.0, "bf16").to(DEV)
    g = synthetic.draw(3, (T, H), "normal", 1.0, "bf16").to(DEV)
    b = synthetic.draw(4, (H,), "normal", 0.02, "bf16").to(DEV)
    gin = synthetic.draw(5, (T, 2 * H), "normal", 1.0, "bf16").to(DEV)
    gb2 = synthetic.draw(6, (2 * H,), "normal", 0.02, "bf16").to(DEV)
    wt = synthetic.draw(7, (T,), "uniform", 1.0, "f32").to(DEV)
    # outputs and workspaces, allocated before capture
    out = {k: torch.empty_like(x) for k in ("bda", "dx", "dgrad", "y", "h", "dxl", "dxs")}
    din = torch.empty_like(gin)
    f32 = lambda n: torch.empty(n, dtype=torch.float32, device=DEV)
    db_bda, db_gelu, db_glu, dw_glu, dg, dbt, dws = f32(H), f32(H), f32(2 * H), f32(T), f32(H), f32(H), f32(T)
    mean, rstd = f32(T), f32(T)
    u8 = lambda n: torch.empty(max(1, n), dtype=torch.uint8, device=DEV)
    ws_bda = u8(mb.mb_bias_dropout_add_bwd_workspace(T, H, x.dtype, True))
    ws_gelu = u8(mb.mb_bias_gelu_bwd_workspace(T, H, x.dtype, True))
    ws_glu = u8(mb.mb_bias_glu_bwd_workspace(T, H, x.dtype, True, True))
    ws_ln = u8(mb.mb_add_layer_norm_bwd_workspace(T, H, x.dtype))
    ws_sr = u8(mb.mb_weighted_squared_relu_bwd_workspace(T, H, x.dtype))

    def step():
        mb.mb_bias_dropout_add_train(x, b, r, 0.1, 77, 5, out=out["bda"])
        mb.mb_bias_dropout_add_bwd(g, 0.1, 77, 5, dx=out["dx"], dresidual=False, dbias=db_bda, ws=ws_bda)
        mb.mb_bias_gelu_bwd(g, x, b, dgrad=out["dgrad"], dbias=db_gelu, ws=ws_gelu)
        mb.mb_bias_swiglu_bwd(g, gin, gb2, wt, din=din, dbias=db_glu, dweights=dw_glu, ws=ws_glu)
        mb.mb_add_layer_norm_fwd(out["bda"], r, b, b, 1e-5, True, h_out=out["h"], y=out["y"], stats=(mean, rstd))
        mb.mb_add_layer_norm_bwd(g, out["h"], b, mean, rstd, True, dh_in=r, dx=out["dxl"], dgamma=dg, dbeta=dbt,
                                 ws=ws_ln)
        mb.mb_weighted_squared_relu_bwd(g, x, wt, dx=out["dxs"], dweights=dws, ws=ws_sr)

    results = lambda: [t.clone() for t in list(out.values()) + [din, db_bda, db_gelu, db_glu, dw_glu, dg, dbt, dws,
                                                                  mean, rstd]]
    step()
    torch.cuda.synchronize()
    eager = results()
    graph = torch.cuda.CUDAGraph()
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()  # warm-up on the side stream, as capture requires
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    with torch.cuda.graph(graph):
        step()
    for rep in range(4):
        for t in list(out.values()) + [din, db_bda, db_gelu, db_glu, dw_glu, dg, dbt, dws, mean, rstd]:
            t.fill_(float("nan") if t.dtype != torch.uint8 else 0)  # eager work between the replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = results()
        for i, (a, e) in enumerate(zip(got, eager)):
            assert torch.equal(bits(a), bits(e)), f"replay {rep}: output {i} differs from the eager run"


@pytest.mark.parametrize("H,in_place,wait", [(16384, False, -1), (32768, False, -1), (32768, False, 0),
                                             (32768, True, -1)],
                         ids=["block", "team", "team-recomputed", "wide-in-place"])
def test_capture_and_replay_wide_layer_norm_backward(H, in_place, wait):
    """The LayerNorm backward of wide rows under capture: 2048 vectors (one
    resident block per CU walking rows), 4096 vectors split over teams of
    blocks (a slot-filling launch, the team kernel, the fix-up launch; also
    with no wait, so every row goes through the fix-up), and 4096 vectors in
    place (the wide-row kernels). Every replay equals the eager result bit
    for bit."""
    T = 300
    dt = "bf16"
    x = synthetic.draw(11, (T, H), "normal", 1.0, dt).to(DEV)
    r = synthetic.draw(12, (T, H), "normal", 1.0, dt).to(DEV)
    g = synthetic.draw(13, (T, H), "normal", 1.0, dt).to(DEV)
    up = synthetic.draw(14, (T, H), "normal", 1.0, dt).to(DEV)
    gm = (synthetic.draw(15, (H,), "normal", 0.3, dt).float() + 1.0).to(torch.bfloat16).to(DEV)
    _, h, mean, rstd = mb.mb_add_layer_norm_fwd(x, r, gm)
    ws = torch.empty(mb.mb_add_layer_norm_bwd_workspace(T, H, x.dtype), dtype=torch.uint8, device=DEV)
    dx, dres = torch.empty_like(x), torch.empty_like(x)
    dg, dbt = (torch.empty(H, dtype=torch.float32, device=DEV) for _ in range(2))
    gi, upi = g.clone(), up.clone()

    def step():
        if in_place:
            gi.copy_(g)
            upi.copy_(up)
            mb.mb_add_layer_norm_bwd(gi, h, gm, mean, rstd, dh_in=upi, dx=gi, dresidual=upi, dgamma=dg, dbeta=dbt,
                                     ws=ws)
        else:
            mb.mb_add_layer_norm_bwd(g, h, gm, mean, rstd, dh_in=up, dx=dx, dresidual=dres, dgamma=dg, dbeta=dbt,
                                     ws=ws)

    outs = (gi, upi, dg, dbt) if in_place else (dx, dres, dg, dbt)
    mb.mb_set_layer_norm_team_wait(wait)
    try:
        step()
        torch.cuda.synchronize()
        eager = [t.clone() for t in outs]
        graph = torch.cuda.CUDAGraph()
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        with torch.cuda.graph(graph):
            step()
        for rep in range(4):
            for t in outs:
                t.fill_(float("nan"))
            ws.fill_(0xA5)  # the launches set their slots and flags themselves
            torch.cuda.synchronize()
            graph.replay()
            torch.cuda.synchronize()
            for i, (a, e) in enumerate(zip(outs, eager)):
                assert torch.equal(bits(a), bits(e)), f"replay {rep}: output {i} differs from the eager run"
    finally:
        mb.mb_set_layer_norm_team_wait(-1)
