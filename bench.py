"""Benchmark of the fused Transformer epilogues on one MI355X.

One step = one pass of every fused op at its full synthetic workload:
  bias-dropout-add, bf16 x [8192, 4096] with fp32 residual, p = 0.1
      (train, its backward with the fp32 residual gradient, and inference in
      place on x), rotating over 4 copies of its tensors so that every call
      streams from HBM (4 x 268 MB exceeds twice the 256 MB last-level cache);
      each in-place inference call gets a fresh copy of x
  bias-SwiGLU fwd + bwd, bf16 [8192, 28672] -> [8192, 14336], unweighted and
      per-token weighted
  bias-GEGLU fwd + bwd, bf16 [16384, 16384] ~ N(0, 2) -> [16384, 8192]
  layer epilogue chain, bf16, 16384 tokens, hidden 8192, ffn 32768, forward
      then backward: attention-out dropout-add -> bias-GeLU -> MLP-out
      dropout-add -> their backward passes in reverse order (dropout-add
      backward regenerates the mask; the residual gradient is g itself)
Inputs are resident in HBM before timing starts. `value` is the algorithmic
bytes of a step (each tensor read or written once, bias and gradients of the
bias included, reduction partials excluded) divided by the step time. The
timed steps replay the step captured into HIP graphs (one per timed step, so
that the rotation above holds; `--eager` times eager launches instead);
per-op durations come from a separate eager loop with HIP events around
every op, which also gives `ms_per_step_eager`.

Every op is also measured against a streaming ceiling (libmb_stream.so): a
kernel with the op's tiling that moves exactly the op's tensors, with the
same pieces per lane and non-temporal loads and stores, and does no
arithmetic; the fastest of a sweep of launch shapes and store forms is the
ceiling, and `frac_ceiling` = ceiling time / op time.

The ops beyond the step (the exact erf GeLU at the chain's MLP shape, the
backward of bias-free layers -- SwiGLU, weighted SwiGLU and the dropout-add
without a bias gradient --, residual add + LayerNorm at hidden 8192, 16384
and 65536, and the MoE weighted squared ReLU) are timed after the step loop,
the same way, and
reported under "next_rows"; the fp32 bias-GeLU at [512, 4096] is timed cold
(48 rotating copies) and warm under "c1". Neither is part of `value`.

The CPU baseline runs the oracle (fp64 C, the parity reference) on the
first rows of every op's inputs, on one pinned core and on a pool of threads
(row chunks), and compares the GPU outputs of those rows with it (per-op
parity statistics); oracle32 (the same formulas in binary32) is timed on the
same rows and the GPU rows' agreement with it reported as a secondary
statistic.

Prints one JSON line (see the keys below). `--gpus N` with N > 1 exits: the
benchmark runs on a single GPU.
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time
from concurrent.futures import ThreadPoolExecutor

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")
TRAFFIC_FILE = os.path.join(PROFILES, "traffic_gelu_bwd_t16384_h32768.json")
STREAM_LIB = os.path.join(ROOT, "transformer_elementwise_epilogues_amd", "libmb_stream.so")
WORKLOAD = "all_epilogues_full_size: bda_bf16_8192x4096_res_f32 (train+bwd+infer, 4 rotating copies) + " \
           "swiglu_bf16_8192x14336 (plain+weighted, fwd+bwd) + geglu_bf16_16384x8192 (fwd+bwd) + " \
           "layer_chain_bf16_t16384_h8192_f32768 (attn bda, gelu, mlp bda: fwd then bwd)"
C2_SETS = 4    # copies of the 268 MB dropout-add working set
C1_SETS = 48   # copies of the 33.6 MB fp32 GeLU working set (1.6 GB)
# the streaming ceiling's sweep: blocks to aim for, rows in flight per wave,
# load and store forms (bit 0: buffer non-temporal stores at system scope,
# else global non-temporal; bit 1: buffer non-temporal loads, else global)
CEIL_BLOCKS = (256, 512, 1024, 2048, 4096, 8192, 16384, 32768, 65536)
CEIL_ROWS = (1, 2, 4)
CEIL_IO = (0, 1, 2, 3)
IO_NAMES = {0: "global nt loads, global nt stores", 1: "global nt loads, buffer nt sc1 stores",
            2: "buffer nt loads, global nt stores", 3: "buffer nt loads, buffer nt sc1 stores"}


def parse(argv=None):
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=30)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--cpu-seconds", type=float, default=8.0,
                    help="target CPU time of each oracle baseline leg (single core, thread pool)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the streaming-ceiling sweep")
    ap.add_argument("--ceiling-table", default=None, help="write every swept shape's time per op to this JSON file")
    ap.add_argument("--eager", action="store_true",
                    help="time the step as eager launches instead of HIP graph replays")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="first copy one 1 GiB buffer device to device (the runtime's copy kernel), so that a "
                         "counter run can scale FETCH_SIZE / WRITE_SIZE by a kernel of known bytes")
    return ap.parse_args(argv)


# ------------------------------------------------------------------ streaming ceiling

class Piece:
    """One tensor of a streaming mix: `rows` rows of `pitch` bytes from byte
    `offset` of `tensor`, of which each lane moves one `piece`-byte piece."""

    def __init__(self, tensor, offset, pitch, piece):
        self.tensor, self.offset, self.pitch, self.piece = tensor, offset, pitch, piece


class Mix:
    """The tensors one op reads and writes, for the streaming-ceiling kernel."""

    def __init__(self, ins, outs, rows, lanes):
        self.ins, self.outs, self.rows, self.lanes = ins, outs, rows, lanes
        self.check()
        self.bytes = rows * lanes * sum(p.piece for p in ins + outs)
        P = ctypes.c_void_p
        self._in = (P * 3)(*[p.tensor.data_ptr() + p.offset for p in ins])
        self._ip = (ctypes.c_int64 * 3)(*[p.pitch for p in ins])
        self._out = (P * 2)(*[p.tensor.data_ptr() + p.offset for p in outs])
        self._op = (ctypes.c_int64 * 2)(*[p.pitch for p in outs])
        self._in8 = sum(1 << i for i, p in enumerate(ins) if p.piece == 8)
        self._out8 = sum(1 << i for i, p in enumerate(outs) if p.piece == 8)

    def check(self):
        """Every lane's piece of every row inside its tensor (checked on the host
        before any launch) and a mix the kernel supports."""
        assert 1 <= len(self.ins) <= 3 and 1 <= len(self.outs) <= 2, "unsupported mix"
        for p in self.ins + self.outs:
            t = p.tensor
            assert t.is_contiguous(), "mix tensors must be contiguous"
            assert p.piece in (8, 16) and p.pitch >= self.lanes * p.piece
            assert (t.data_ptr() + p.offset) % 16 == 0 and p.pitch % p.piece == 0
            end = p.offset + (self.rows - 1) * p.pitch + self.lanes * p.piece
            assert end <= t.numel() * t.element_size(), "mix piece beyond its tensor"
        in8 = [p.piece for p in self.ins]
        out8 = [p.piece for p in self.outs]
        assert (set(in8) == {16} and set(out8) == {16}) or (in8, out8) in (([8, 16], [8]), ([8], [8, 16])), \
            "unsupported piece sizes"

    def launch(self, lib, blocks, rows_in_flight, io, stream):
        rc = lib.mbs_stream(self._in, self._ip, len(self.ins), self._in8, self._out, self._op, len(self.outs),
                            self._out8, self.rows, self.lanes, blocks, rows_in_flight, io, stream)
        if rc != 0:
            raise RuntimeError(f"mbs_stream returned {rc}")


def stream_lib():
    if not os.path.exists(STREAM_LIB):
        raise RuntimeError(f"{STREAM_LIB} is not built: run `python -m transformer_elementwise_epilogues_amd.build_lib`")
    L = ctypes.CDLL(STREAM_LIB)
    P, I, U, I64 = ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_int64
    L.mbs_stream.argtypes = [P, P, I, U, P, P, I, U, I64, I, I, I, I, P]
    L.mbs_stream.restype = I
    return L


def rows_mix(ins, outs, rows, row_bytes):
    """Whole rows of row_bytes from each tensor in 16-byte pieces."""
    return Mix([Piece(t, 0, row_bytes, 16) for t in ins], [Piece(t, 0, row_bytes, 16) for t in outs], rows,
               row_bytes // 16)


def glu_fwd_mix(inp, out):
    """a and b, the two halves of each input row, to the output row."""
    T, H2 = inp.shape
    hb = H2 // 2 * inp.element_size()
    return Mix([Piece(inp, 0, 2 * hb, 16), Piece(inp, hb, 2 * hb, 16)], [Piece(out, 0, hb, 16)], T, hb // 16)


def glu_bwd_mix(g, inp, din):
    T, H2 = inp.shape
    hb = H2 // 2 * inp.element_size()
    return Mix([Piece(g, 0, hb, 16), Piece(inp, 0, 2 * hb, 16), Piece(inp, hb, 2 * hb, 16)],
               [Piece(din, 0, 2 * hb, 16), Piece(din, hb, 2 * hb, 16)], T, hb // 16)


# ------------------------------------------------------------------ the ops

class Op:
    """A timed op: call k runs calls[k % len(calls)] (rotating buffer sets);
    mixes likewise for its streaming ceiling; refresh() restores inputs that
    in-place calls overwrote; outputs() names the output tensors of call 0
    that the parity statistics compare."""

    def __init__(self, name, nbytes, kernels, calls, mixes, outputs, refresh=None):
        self.name, self.nbytes, self.kernels = name, nbytes, kernels
        self.calls, self.mixes, self.outputs, self.refresh = calls, mixes, outputs, refresh
        self.ms = []

    def call(self, k):
        self.calls[k % len(self.calls)]()


def build_ops(dev, ncopies):
    import torch

    import transformer_elementwise_epilogues_amd as mb
    from transformer_elementwise_epilogues_amd.synthetic import WORKLOADS

    f32 = torch.float32
    host = {}  # CPU copies for the oracle baseline
    ops = []

    def load(wname, tname):
        t = WORKLOADS[wname].tensor(tname)
        host[(wname, tname)] = t
        return t.to(dev)

    def ws_of(n):
        return torch.empty(max(1, n), dtype=torch.uint8, device=dev)

    # -- bias-dropout-add, bf16 with fp32 residual: C2_SETS copies of every tensor
    w = WORKLOADS["bda_bf16_8192x4096_res_f32"]
    x, b, r, g = (load(w.name, k) for k in ("x", "bias", "residual", "g"))
    T, H = x.shape
    S = [dict(x=x, b=b, r=r, g=g)] + [dict(x=x.clone(), b=b.clone(), r=r.clone(), g=g.clone())
                                      for _ in range(C2_SETS - 1)]
    for s in S:
        s.update(out=torch.empty_like(x), dx=torch.empty_like(x), dr=torch.empty_like(r),
                 db=torch.empty(H, dtype=f32, device=dev),
                 ws=ws_of(mb.mb_bias_dropout_add_bwd_workspace(T, H, x.dtype, True)))
    xi = [torch.empty_like(x) for _ in range(ncopies)]  # a fresh x for every in-place inference call

    def refresh_xi():
        for k, t in enumerate(xi):
            t.copy_(S[k % C2_SETS]["x"])

    p, seed, off = w.params["p"], w.params["seed"], w.params["offset"]
    bda_bytes = T * H * (2 + 4 + 2) + H * 2
    lanes = H // 4  # 4 elements per lane beside the fp32 residual: 8-byte x pieces, 16-byte residual pieces

    def bda_mix(s, xt, ot):
        return Mix([Piece(xt, 0, H * 2, 8), Piece(s["r"], 0, H * 4, 16)], [Piece(ot, 0, H * 2, 8)], T, lanes)

    refresh_xi()
    ops.append(Op("bda_train_bf16_res_f32_8192x4096", bda_bytes, ["bda"],
                  [lambda s=s: mb.mb_bias_dropout_add_train(s["x"], s["b"], s["r"], p, seed, off, out=s["out"])
                   for s in S],
                  [bda_mix(s, s["x"], s["out"]) for s in S], {"out": S[0]["out"]}))
    ops.append(Op("bda_bwd_bf16_res_f32_8192x4096", T * H * (2 + 2 + 4) + H * 4, ["bda_bwd", "colsum"],
                  [lambda s=s: mb.mb_bias_dropout_add_bwd(s["g"], p, seed, off, residual_dtype=f32, dx=s["dx"],
                                                          dresidual=s["dr"], dbias=s["db"], ws=s["ws"])
                   for s in S],
                  [Mix([Piece(s["g"], 0, H * 2, 8)], [Piece(s["dx"], 0, H * 2, 8), Piece(s["dr"], 0, H * 4, 16)],
                       T, lanes) for s in S],
                  {"dx": S[0]["dx"], "dresidual": S[0]["dr"]}))
    # the inference call of step k reads the residual of set k + 2, which the
    # training pass of step k did not just stream
    ops.append(Op("bda_infer_inplace_bf16_res_f32_8192x4096", bda_bytes, ["bda"],
                  [lambda k=k: mb.mb_bias_dropout_add_infer(xi[k], S[(k + 2) % C2_SETS]["b"],
                                                            S[(k + 2) % C2_SETS]["r"], out=xi[k])
                   for k in range(ncopies)],
                  [bda_mix(S[(k + 2) % C2_SETS], xi[k], xi[k]) for k in range(ncopies)], {"out": xi[0]},
                  refresh=refresh_xi))

    # -- SwiGLU, plain and weighted
    w = WORKLOADS["swiglu_bf16_8192x14336"]
    xin, b2, g3, wt = (load(w.name, k) for k in ("in", "bias", "g", "weights"))
    T, H2 = xin.shape
    H = H2 // 2
    o3 = torch.empty((T, H), dtype=xin.dtype, device=dev)
    din3 = torch.empty_like(xin)
    db3 = torch.empty(2 * H, dtype=f32, device=dev)
    dw3 = torch.empty(T, dtype=f32, device=dev)
    ws3 = ws_of(mb.mb_bias_glu_bwd_workspace(T, H, xin.dtype, True, True))
    fwd_b = T * H * 3 * 2 + 2 * H * 2
    bwd_b = T * H * 5 * 2 + 2 * H * 2 + 2 * H * 4
    fm, bm = glu_fwd_mix(xin, o3), glu_bwd_mix(g3, xin, din3)
    ops.append(Op("swiglu_fwd_bf16_8192x14336", fwd_b, ["glu_fwd"],
                  [lambda: mb.mb_bias_swiglu_fwd(xin, b2, out=o3)], [fm], {"out": o3}))
    ops.append(Op("swiglu_bwd_bf16_8192x14336", bwd_b, ["glu_bwd", "colsum"],
                  [lambda: mb.mb_bias_swiglu_bwd(g3, xin, b2, din=din3, dbias=db3, dweights=False, ws=ws3)], [bm],
                  {"din": din3}))
    ops.append(Op("weighted_swiglu_fwd_bf16_8192x14336", fwd_b + T * 2, ["glu_fwd"],
                  [lambda: mb.mb_bias_swiglu_fwd(xin, b2, wt, out=o3)], [fm], {"out": o3}))
    ops.append(Op("weighted_swiglu_bwd_bf16_8192x14336", bwd_b + T * 2 + T * 4, ["glu_bwd", "colsum"],
                  [lambda: mb.mb_bias_swiglu_bwd(g3, xin, b2, wt, din=din3, dbias=db3, dweights=dw3, ws=ws3)], [bm],
                  {"din": din3, "dweights": dw3}))

    # -- GEGLU
    w = WORKLOADS["geglu_bf16_16384x8192"]
    xin4, b4, g4 = (load(w.name, k) for k in ("in", "bias", "g"))
    T, H2 = xin4.shape
    H = H2 // 2
    o4 = torch.empty((T, H), dtype=xin4.dtype, device=dev)
    din4 = torch.empty_like(xin4)
    db4 = torch.empty(2 * H, dtype=f32, device=dev)
    ws4 = ws_of(mb.mb_bias_glu_bwd_workspace(T, H, xin4.dtype, True, False))
    ops.append(Op("geglu_fwd_bf16_16384x8192", T * H * 3 * 2 + 2 * H * 2, ["glu_fwd"],
                  [lambda: mb.mb_bias_geglu_fwd(xin4, b4, out=o4)], [glu_fwd_mix(xin4, o4)], {"out": o4}))
    ops.append(Op("geglu_bwd_bf16_16384x8192", T * H * 5 * 2 + 2 * H * 2 + 2 * H * 4, ["glu_bwd", "colsum"],
                  [lambda: mb.mb_bias_geglu_bwd(g4, xin4, b4, din=din4, dbias=db4, ws=ws4)],
                  [glu_bwd_mix(g4, xin4, din4)], {"din": din4}))

    # -- layer epilogue chain
    w = WORKLOADS["layer_chain_bf16_t16384_h8192_f32768"]
    ax, ar, ab, ag = (load(w.name, k) for k in ("attn_x", "attn_residual", "attn_bias", "attn_g"))
    gy, gb, gg = (load(w.name, k) for k in ("gelu_y", "gelu_bias", "gelu_g"))
    mx, mr, mbias, mg = (load(w.name, k) for k in ("mlp_x", "mlp_residual", "mlp_bias", "mlp_g"))
    aout, mout = torch.empty_like(ax), torch.empty_like(mx)
    adx, mdx = torch.empty_like(ax), torch.empty_like(mx)
    gout, dgr = torch.empty_like(gy), torch.empty_like(gy)
    T, H = gy.shape
    dbg = torch.empty(H, dtype=f32, device=dev)
    wsg = ws_of(mb.mb_bias_gelu_bwd_workspace(T, H, gy.dtype, True))
    Ta, Ha = ax.shape
    adb, mdb = (torch.empty(Ha, dtype=f32, device=dev) for _ in range(2))
    wsb = ws_of(mb.mb_bias_dropout_add_bwd_workspace(Ta, Ha, ax.dtype, True))
    p5, s_attn, s_mlp, off5 = w.params["p"], w.params["attn_seed"], w.params["mlp_seed"], w.params["offset"]
    bda5 = Ta * Ha * 6 + Ha * 2
    bwd5 = Ta * Ha * 4 + Ha * 4  # read g, write dx, dbias; the residual gradient is g itself
    ops.append(Op("chain_attn_bda_train_bf16_16384x8192", bda5, ["bda"],
                  [lambda: mb.mb_bias_dropout_add_train(ax, ab, ar, p5, s_attn, off5, out=aout)],
                  [rows_mix([ax, ar], [aout], Ta, Ha * 2)], {"out": aout}))
    ops.append(Op("chain_gelu_fwd_bf16_16384x32768", T * H * 4 + H * 2, ["gelu_fwd"],
                  [lambda: mb.mb_bias_gelu_fwd(gy, gb, out=gout)], [rows_mix([gy], [gout], T, H * 2)],
                  {"out": gout}))
    ops.append(Op("chain_mlp_bda_train_bf16_16384x8192", bda5, ["bda"],
                  [lambda: mb.mb_bias_dropout_add_train(mx, mbias, mr, p5, s_mlp, off5, out=mout)],
                  [rows_mix([mx, mr], [mout], Ta, Ha * 2)], {"out": mout}))
    ops.append(Op("chain_mlp_bda_bwd_bf16_16384x8192", bwd5, ["bda_bwd", "colsum"],
                  [lambda: mb.mb_bias_dropout_add_bwd(mg, p5, s_mlp, off5, dx=mdx, dresidual=False, dbias=mdb,
                                                      ws=wsb)],
                  [rows_mix([mg], [mdx], Ta, Ha * 2)], {"dx": mdx}))
    ops.append(Op("chain_gelu_bwd_bf16_16384x32768", T * H * 6 + H * 2 + H * 4, ["gelu_bwd", "colsum_fold"],
                  [lambda: mb.mb_bias_gelu_bwd(gg, gy, gb, dgrad=dgr, dbias=dbg, ws=wsg)],
                  [rows_mix([gg, gy], [dgr], T, H * 2)], {"dgrad": dgr}))
    ops.append(Op("chain_attn_bda_bwd_bf16_16384x8192", bwd5, ["bda_bwd", "colsum"],
                  [lambda: mb.mb_bias_dropout_add_bwd(ag, p5, s_attn, off5, dx=adx, dresidual=False, dbias=adb,
                                                      ws=wsb)],
                  [rows_mix([ag], [adx], Ta, Ha * 2)], {"dx": adx}))

    # -- beyond the step: the exact (erf) GeLU on the chain's MLP activation
    wse = ws_of(mb.mb_bias_gelu_erf_bwd_workspace(T, H, gy.dtype, True))
    extra = [Op("erf_gelu_fwd_bf16_16384x32768", T * H * 4 + H * 2, ["gelu_fwd"],
                [lambda: mb.mb_bias_gelu_erf_fwd(gy, gb, out=gout)], [rows_mix([gy], [gout], T, H * 2)],
                {"out": gout}),
             Op("erf_gelu_bwd_bf16_16384x32768", T * H * 6 + H * 2 + H * 4, ["gelu_bwd", "colsum_fold"],
                [lambda: mb.mb_bias_gelu_erf_bwd(gg, gy, gb, dgrad=dgr, dbias=dbg, ws=wse)],
                [rows_mix([gg, gy], [dgr], T, H * 2)], {"dgrad": dgr})]

    # -- beyond the step: the backward of bias-free layers (no bias gradient, so
    # no partial rows: each takes its own many-block launch shape)
    T3 = xin.shape[0]
    H3 = xin.shape[1] // 2
    extra.append(Op("swiglu_bwd_nobias_bf16_8192x14336", T3 * H3 * 10, ["glu_bwd"],
                    [lambda: mb.mb_bias_swiglu_bwd(g3, xin, None, din=din3, dbias=False, dweights=False)],
                    [glu_bwd_mix(g3, xin, din3)], {"din": din3}))
    extra.append(Op("weighted_swiglu_bwd_nobias_bf16_8192x14336", T3 * H3 * 10 + T3 * 6, ["glu_bwd", "colsum"],
                    [lambda: mb.mb_bias_swiglu_bwd(g3, xin, None, wt, din=din3, dbias=False, dweights=dw3, ws=ws3)],
                    [glu_bwd_mix(g3, xin, din3)], {"din": din3, "dweights": dw3}))
    extra.append(Op("chain_mlp_bda_bwd_nodbias_bf16_16384x8192", Ta * Ha * 4, ["bda_bwd"],
                    [lambda: mb.mb_bias_dropout_add_bwd(mg, p5, s_mlp, off5, dx=mdx, dresidual=False, dbias=False)],
                    [rows_mix([mg], [mdx], Ta, Ha * 2)], {"dx": mdx}))

    # -- beyond the step: residual add + LayerNorm, bf16, hidden 8192, 16384 and 65536
    for wname in ("add_ln_bf16_16384x8192", "add_ln_bf16_8192x16384", "add_ln_bf16_2048x65536"):
        w = WORKLOADS[wname]
        lx, lr, lg, lb, ldy, lup = (load(w.name, k) for k in ("x", "residual", "gamma", "beta", "dy", "dh_in"))
        T, H = lx.shape
        lh, ly, ldx = torch.empty_like(lx), torch.empty_like(lx), torch.empty_like(lx)
        lmean, lrstd = (torch.empty(T, dtype=f32, device=dev) for _ in range(2))
        ldg, ldb = (torch.empty(H, dtype=f32, device=dev) for _ in range(2))
        lws = ws_of(mb.mb_add_layer_norm_bwd_workspace(T, H, lx.dtype))
        eps, zc = w.params["eps"], w.params["zero_centered_gamma"]
        tag = wname[len("add_ln_"):]
        extra.append(Op(f"add_ln_fwd_{tag}", T * H * 8 + H * 4 + T * 8, ["ln_fwd"],
                        [lambda lx=lx, lr=lr, lg=lg, lb=lb, eps=eps, zc=zc, lh=lh, ly=ly, lmean=lmean, lrstd=lrstd:
                         mb.mb_add_layer_norm_fwd(lx, lr, lg, lb, eps, zc, h_out=lh, y=ly, stats=(lmean, lrstd))],
                        [rows_mix([lx, lr], [lh, ly], T, H * 2)], {"h": lh, "y": ly}))
        extra.append(Op(f"add_ln_bwd_{tag}", T * H * 8 + H * 2 + T * 8 + H * 8, ["ln_bwd", "colsum"],
                        [lambda ldy=ldy, lh=lh, lg=lg, lmean=lmean, lrstd=lrstd, zc=zc, lup=lup, ldx=ldx, ldg=ldg,
                         ldb=ldb, lws=lws:
                         mb.mb_add_layer_norm_bwd(ldy, lh, lg, lmean, lrstd, zc, dh_in=lup, dx=ldx, dgamma=ldg,
                                                  dbeta=ldb, ws=lws)],
                        [rows_mix([ldy, lh, lup], [ldx], T, H * 2)], {"dx": ldx}))

    # -- beyond the step: MoE weighted squared ReLU, bf16 [8192, 14336], fp32 weights
    w = WORKLOADS["wsrelu_bf16_8192x14336"]
    sx, sg, sw = (load(w.name, k) for k in ("x", "g", "weights"))
    T, H = sx.shape
    so, sdx = torch.empty_like(sx), torch.empty_like(sx)
    sdw = torch.empty(T, dtype=f32, device=dev)
    sws = ws_of(mb.mb_weighted_squared_relu_bwd_workspace(T, H, sx.dtype))
    extra.append(Op("weighted_squared_relu_fwd_bf16_8192x14336", T * H * 4 + T * 4, ["srelu_fwd"],
                    [lambda: mb.mb_weighted_squared_relu_fwd(sx, sw, out=so)], [rows_mix([sx], [so], T, H * 2)],
                    {"out": so}))
    extra.append(Op("weighted_squared_relu_bwd_bf16_8192x14336", T * H * 6 + T * 8, ["srelu_bwd", "colsum"],
                    [lambda: mb.mb_weighted_squared_relu_bwd(sg, sx, sw, dx=sdx, dweights=sdw, ws=sws)],
                    [rows_mix([sg, sx], [sdx], T, H * 2)], {"dx": sdx, "dweights": sdw}))
    return ops, extra, host


# ------------------------------------------------------------------ timing

def log(msg):
    """Progress of the run on stderr (stdout carries only the JSON line)."""
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def events(n):
    import torch

    return [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]


def time_calls(fn, n, stream):
    """Average ms of fn(i) for i < n, each bracketed by HIP events on `stream`."""
    import torch

    ev = events(n)
    for i, (e0, e1) in enumerate(ev):
        e0.record(stream)
        fn(i)
        e1.record(stream)
    torch.cuda.synchronize()
    return sum(e0.elapsed_time(e1) for e0, e1 in ev) / n


def ceiling(op, L, stream, table=None, finalists=3):
    """Fastest streaming of the op's mix over the sweep: a short run per shape,
    then the `finalists` fastest shapes again over more launches, the fastest
    of those kept (a single short run of a persistent grid varies by several
    per cent between calls). table (a dict) receives every shape's time."""
    s = ctypes.c_void_p(stream.cuda_stream)
    nm = len(op.mixes)

    def run(shape, n):
        blocks, u, io = shape
        return time_calls(lambda i: op.mixes[i % nm].launch(L, blocks, u, io, s), n, stream)

    sweep = []
    for shape in ((b, u, io) for b in CEIL_BLOCKS for u in CEIL_ROWS for io in CEIL_IO):
        run(shape, 1)
        ms = run(shape, max(6, nm))
        if table is not None:
            table[f"{shape[0]}x{shape[1]}/{shape[2]}"] = round(ms * 1e3, 2)
        sweep.append((ms, shape))
    sweep.sort(key=lambda x: x[0])
    ms, shape = min((run(sh, max(24, 2 * nm)), sh) for _, sh in sweep[:finalists])
    blocks, u, io = shape
    return {"us": round(ms * 1e3, 2), "gbs": round(op.mixes[0].bytes / (ms * 1e-3) / 1e9, 1), "blocks": blocks,
            "rows_in_flight": u, "io": IO_NAMES[io]}


def c1_bench(dev, L, stream, sweep):
    """The fp32 bias-GeLU at [512, 4096] (a correctness-sized workload whose
    tensors fit the last-level cache): forward and backward timed cold, rotating
    over C1_SETS copies of the inputs and outputs, and warm, on one copy, as
    graphs of C1_SETS launches; the same for the streaming ceiling."""
    import torch

    import transformer_elementwise_epilogues_amd as mb
    from transformer_elementwise_epilogues_amd.synthetic import WORKLOADS

    w = WORKLOADS["gelu_f32_512x4096"]
    y0, b, g0 = (w.tensor(k).to(dev) for k in ("y", "bias", "g"))
    T, H = y0.shape
    ys = [y0] + [y0.clone() for _ in range(C1_SETS - 1)]
    gs = [g0] + [g0.clone() for _ in range(C1_SETS - 1)]
    outs = [torch.empty_like(y0) for _ in range(C1_SETS)]
    dgs = [torch.empty_like(y0) for _ in range(C1_SETS)]
    dbs = [torch.empty(H, dtype=torch.float32, device=dev) for _ in range(C1_SETS)]
    nws = max(1, mb.mb_bias_gelu_bwd_workspace(T, H, torch.float32, True))
    wss = [torch.empty(nws, dtype=torch.uint8, device=dev) for _ in range(C1_SETS)]
    def cur():
        return ctypes.c_void_p(torch.cuda.current_stream(dev).cuda_stream)

    def graph_us(fn):
        """µs per launch of fn(i), i < C1_SETS, captured once into a graph and
        replayed (median of 9 replays)."""
        side = torch.cuda.Stream(dev)
        side.wait_stream(stream)
        with torch.cuda.stream(side):
            for i in range(C1_SETS):
                fn(i)
        stream.wait_stream(side)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for i in range(C1_SETS):
                fn(i)
        for _ in range(2):
            gr.replay()
        torch.cuda.synchronize()
        ev = events(9)
        for e0, e1 in ev:
            e0.record(stream)
            gr.replay()
            e1.record(stream)
        torch.cuda.synchronize()
        t = sorted(e0.elapsed_time(e1) for e0, e1 in ev)[4]
        return t * 1e3 / C1_SETS

    fwd_mix = [rows_mix([ys[i]], [outs[i]], T, H * 4) for i in range(C1_SETS)]
    bwd_mix = [rows_mix([gs[i], ys[i]], [dgs[i]], T, H * 4) for i in range(C1_SETS)]
    res = {}
    for name, nbytes, cold, warm, mixes in (
            ("gelu_fwd_f32_512x4096", T * H * 8 + H * 4,
             lambda i: mb.mb_bias_gelu_fwd(ys[i], b, out=outs[i]),
             lambda i: mb.mb_bias_gelu_fwd(ys[0], b, out=outs[0]), fwd_mix),
            ("gelu_bwd_f32_512x4096", T * H * 12 + H * 8,
             lambda i: mb.mb_bias_gelu_bwd(gs[i], ys[i], b, dgrad=dgs[i], dbias=dbs[i], ws=wss[i]),
             lambda i: mb.mb_bias_gelu_bwd(gs[0], ys[0], b, dgrad=dgs[0], dbias=dbs[0], ws=wss[0]), bwd_mix)):
        r = {"bytes": nbytes}
        for kind, fn in (("cold", cold), ("warm", warm)):
            us = graph_us(fn)
            r[f"{kind}_us"] = round(us, 3)
            r[f"{kind}_gbs"] = round(nbytes / (us * 1e-6) / 1e9, 1)
        r["frac_peak_cold"] = round(r["cold_gbs"] / PEAK_HBM_GBS, 4)
        if sweep:
            for kind in ("cold", "warm"):
                best = None
                for shape in ((bl, u, io) for bl in (256, 1024, 4096, 16384) for u in (1, 2) for io in CEIL_IO):
                    pick = (lambda i, shape=shape: mixes[i].launch(L, *shape, cur())) if kind == "cold" else \
                        (lambda i, shape=shape: mixes[0].launch(L, *shape, cur()))
                    us = graph_us(pick)
                    best = us if best is None or us < best else best
                r[f"ceiling_{kind}_us"] = round(best, 3)
                r[f"frac_ceiling_{kind}"] = round(best / r[f"{kind}_us"], 4)
        res[name] = r
    return res


# ------------------------------------------------------------------ traffic counters

def source_hash(files):
    h = hashlib.sha256()
    for f in files:
        with open(os.path.join(ROOT, f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


TRAFFIC_SOURCES = ["transformer_elementwise_epilogues_amd/csrc/mb_gelu.hip",
                   "transformer_elementwise_epilogues_amd/csrc/mb_device.hpp",
                   "transformer_elementwise_epilogues_amd/csrc/mb_reduce.hip",
                   "transformer_elementwise_epilogues_amd/csrc/mb_launch.hpp",
                   "transformer_elementwise_epilogues_amd/csrc/mb_plan.hpp",
                   "transformer_elementwise_epilogues_amd/csrc/mb_plan.cpp",
                   "transformer_elementwise_epilogues_amd/csrc/mb_abi.cpp"]


def measured_traffic():
    """HBM bytes per launch of the dominant op from the committed rocprofv3 counter
    summary, or None when it is missing or the kernel sources changed since."""
    try:
        with open(TRAFFIC_FILE) as fh:
            t = json.load(fh)
    except (OSError, ValueError):
        return None
    if t.get("source_hash") != source_hash(TRAFFIC_SOURCES):
        return None
    return t.get("bytes_per_launch")


# ------------------------------------------------------------------ CPU baseline and parity statistics

def cpu_info():
    """The host CPU as /proc/cpuinfo names it (a virtualised host may give only
    a family name; vendor, family and model number identify the core)."""
    fields = {"model name": "model", "vendor_id": "vendor", "cpu family": "family", "model": "model_number",
              "cpu MHz": "mhz", "cache size": "cache"}
    info = {v: None for v in fields.values()}
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if not line.strip():
                    break  # the first processor's block is enough
                key, _, val = line.partition(":")
                if key.strip() in fields:
                    info[fields[key.strip()]] = val.strip()
    except OSError:
        pass
    try:
        avail = len(os.sched_getaffinity(0))
    except AttributeError:
        avail = os.cpu_count() or 1
    info.update({"nproc": os.cpu_count(), "available": avail})
    return info


def oracle_plan(host):
    """Per op name: (oracle over rows [r0, r1) -> {output: (kind, expected...)},
    algorithmic bytes of n rows, rows of the op, oracle32 over rows [r0, r1) ->
    {output: storage}). Kinds: "elem" (storage, o64, mag), "bounded"
    (storage, o64, bound), "exact" (storage), "rowsum" (o64)."""
    import numpy as np

    import oracle
    from oracle import oracle32
    from oracle.tolerances import to_storage

    def rows(w, t, r0, r1):
        return to_storage(host[(w, t)][r0:r1])

    def vec(w, t):
        return to_storage(host[(w, t)])

    c2, c3, c4, c5 = ("bda_bf16_8192x4096_res_f32", "swiglu_bf16_8192x14336", "geglu_bf16_16384x8192",
                      "layer_chain_bf16_t16384_h8192_f32768")
    plan = {}

    def bda(w, xn, bn, rn, rdt, train, p, seed):
        def f(r0, r1):
            o, o64, mag = oracle.bias_dropout_add("bf16", rows(w, xn, r0, r1), vec(w, bn), rows(w, rn, r0, r1), rdt,
                                                  train, p, seed, 0, row0=r0)
            return {"out": ("elem", o, o64, mag)}
        return f

    def bda_bwd(w, gn, rdt, p, seed, want_dres):
        def f(r0, r1):
            dx, dx64, dres, _ = oracle.bias_dropout_add_bwd("bf16", rows(w, gn, r0, r1), rdt, p, seed, 0, row0=r0,
                                                            want_dres=want_dres)
            res = {"dx": ("elem", dx, dx64, None)}
            if want_dres:
                res["dresidual"] = ("exact", dres)
            return res
        return f

    # oracle32: the same rows in binary32, the secondary statistic and the fp32 CPU baseline
    plan32 = {}

    def bda32(w, xn, bn, rn, rdt, train, p, seed):
        return lambda r0, r1: {"out": oracle32.bias_dropout_add("bf16", rows(w, xn, r0, r1), vec(w, bn),
                                                                rows(w, rn, r0, r1), rdt, train, p, seed, 0, row0=r0)}

    def bda_bwd32(w, gn, rdt, p, seed):
        return lambda r0, r1: {"dx": oracle32.bias_dropout_add_bwd("bf16", rows(w, gn, r0, r1), rdt, p, seed, 0,
                                                                   row0=r0, want_dres=False)[0]}

    plan32["bda_train_bf16_res_f32_8192x4096"] = bda32(c2, "x", "bias", "residual", "f32", True, 0.1, 1234)
    plan32["bda_bwd_bf16_res_f32_8192x4096"] = bda_bwd32(c2, "g", "f32", 0.1, 1234)
    plan32["bda_infer_inplace_bf16_res_f32_8192x4096"] = bda32(c2, "x", "bias", "residual", "f32", False, 0.0, 0)
    plan32["chain_attn_bda_train_bf16_16384x8192"] = bda32(c5, "attn_x", "attn_bias", "attn_residual", "bf16", True,
                                                           0.1, 5001)
    plan32["chain_mlp_bda_train_bf16_16384x8192"] = bda32(c5, "mlp_x", "mlp_bias", "mlp_residual", "bf16", True, 0.1,
                                                          5002)
    plan32["chain_mlp_bda_bwd_bf16_16384x8192"] = bda_bwd32(c5, "mlp_g", "bf16", 0.1, 5002)
    plan32["chain_attn_bda_bwd_bf16_16384x8192"] = bda_bwd32(c5, "attn_g", "bf16", 0.1, 5001)

    def glu32(w, act, wt, bwd, bias=True):
        def f(r0, r1):
            wts = None if wt is None else rows(w, wt, r0, r1)
            if bwd:
                return {"din": oracle32.bias_glu_bwd(act, "bf16", rows(w, "g", r0, r1), rows(w, "in", r0, r1),
                                                     vec(w, "bias") if bias else None, wts)[0]}
            return {"out": oracle32.bias_glu_fwd(act, "bf16", rows(w, "in", r0, r1), vec(w, "bias"), wts)}
        return f

    for name, wt in (("swiglu", None), ("weighted_swiglu", "weights")):
        plan32[f"{name}_fwd_bf16_8192x14336"] = glu32(c3, "swiglu", wt, False)
        plan32[f"{name}_bwd_bf16_8192x14336"] = glu32(c3, "swiglu", wt, True)
        plan32[f"{name}_bwd_nobias_bf16_8192x14336"] = glu32(c3, "swiglu", wt, True, bias=False)
    plan32["chain_mlp_bda_bwd_nodbias_bf16_16384x8192"] = bda_bwd32(c5, "mlp_g", "bf16", 0.1, 5002)
    plan32["geglu_fwd_bf16_16384x8192"] = glu32(c4, "geglu", None, False)
    plan32["geglu_bwd_bf16_16384x8192"] = glu32(c4, "geglu", None, True)

    def gelu32(exact, bwd):
        def f(r0, r1):
            y, b = rows(c5, "gelu_y", r0, r1), vec(c5, "gelu_bias")
            if bwd:
                return {"dgrad": oracle32.bias_gelu_bwd("bf16", rows(c5, "gelu_g", r0, r1), y, b, exact=exact)[0]}
            return {"out": oracle32.bias_gelu_fwd("bf16", y, b, exact=exact)}
        return f

    plan32["chain_gelu_fwd_bf16_16384x32768"] = gelu32(False, False)
    plan32["chain_gelu_bwd_bf16_16384x32768"] = gelu32(False, True)
    plan32["erf_gelu_fwd_bf16_16384x32768"] = gelu32(True, False)
    plan32["erf_gelu_bwd_bf16_16384x32768"] = gelu32(True, True)

    plan["bda_train_bf16_res_f32_8192x4096"] = (bda(c2, "x", "bias", "residual", "f32", True, 0.1, 1234),
                                                lambda n: n * 4096 * 8 + 4096 * 2)
    plan["bda_bwd_bf16_res_f32_8192x4096"] = (bda_bwd(c2, "g", "f32", 0.1, 1234, True),
                                              lambda n: n * 4096 * 8 + 4096 * 4)
    plan["bda_infer_inplace_bf16_res_f32_8192x4096"] = (bda(c2, "x", "bias", "residual", "f32", False, 0.0, 0),
                                                        lambda n: n * 4096 * 8 + 4096 * 2)

    def glu_fwd(w, act, wt):
        def f(r0, r1):
            o, o64 = oracle.bias_glu_fwd(act, "bf16", rows(w, "in", r0, r1), vec(w, "bias"),
                                         None if wt is None else rows(w, wt, r0, r1))
            return {"out": ("elem", o, o64, None)}
        return f

    def glu_bwd(w, act, wt, bias=True):
        def f(r0, r1):
            d, d64, mag, _, dw = oracle.bias_glu_bwd(act, "bf16", rows(w, "g", r0, r1), rows(w, "in", r0, r1),
                                                     vec(w, "bias") if bias else None,
                                                     None if wt is None else rows(w, wt, r0, r1))
            res = {"din": ("elem", d, d64, mag)}
            if dw is not None:
                res["dweights"] = ("rowsum", dw)
            return res
        return f

    for name, wt in (("swiglu", None), ("weighted_swiglu", "weights")):
        plan[f"{name}_fwd_bf16_8192x14336"] = (glu_fwd(c3, "swiglu", wt), lambda n: n * 14336 * 6 + 28672 * 2)
        plan[f"{name}_bwd_bf16_8192x14336"] = (glu_bwd(c3, "swiglu", wt), lambda n: n * 14336 * 10 + 28672 * 6)
        plan[f"{name}_bwd_nobias_bf16_8192x14336"] = (glu_bwd(c3, "swiglu", wt, bias=False),
                                                      (lambda n: n * 14336 * 10) if wt is None
                                                      else (lambda n: n * 14336 * 10 + n * 6))
    plan["geglu_fwd_bf16_16384x8192"] = (glu_fwd(c4, "geglu", None), lambda n: n * 8192 * 6 + 16384 * 2)
    plan["geglu_bwd_bf16_16384x8192"] = (glu_bwd(c4, "geglu", None), lambda n: n * 8192 * 10 + 16384 * 6)

    def gelu_fwd(exact):
        def f(r0, r1):
            o, o64 = oracle.bias_gelu_fwd("bf16", rows(c5, "gelu_y", r0, r1), vec(c5, "gelu_bias"), exact=exact)
            return {"out": ("elem", o, o64, None)}
        return f

    def gelu_bwd(exact):
        def f(r0, r1):
            d, d64, mag, _ = oracle.bias_gelu_bwd("bf16", rows(c5, "gelu_g", r0, r1), rows(c5, "gelu_y", r0, r1),
                                                  vec(c5, "gelu_bias"), exact=exact)
            return {"dgrad": ("elem", d, d64, mag)}
        return f

    plan["chain_attn_bda_train_bf16_16384x8192"] = (bda(c5, "attn_x", "attn_bias", "attn_residual", "bf16", True, 0.1,
                                                        5001), lambda n: n * 8192 * 6 + 8192 * 2)
    plan["chain_gelu_fwd_bf16_16384x32768"] = (gelu_fwd(False), lambda n: n * 32768 * 4 + 32768 * 2)
    plan["chain_mlp_bda_train_bf16_16384x8192"] = (bda(c5, "mlp_x", "mlp_bias", "mlp_residual", "bf16", True, 0.1,
                                                       5002), lambda n: n * 8192 * 6 + 8192 * 2)
    plan["chain_mlp_bda_bwd_bf16_16384x8192"] = (bda_bwd(c5, "mlp_g", "bf16", 0.1, 5002, False),
                                                 lambda n: n * 8192 * 4 + 8192 * 4)
    plan["chain_gelu_bwd_bf16_16384x32768"] = (gelu_bwd(False), lambda n: n * 32768 * 6 + 32768 * 6)
    plan["chain_mlp_bda_bwd_nodbias_bf16_16384x8192"] = (bda_bwd(c5, "mlp_g", "bf16", 0.1, 5002, False),
                                                         lambda n: n * 8192 * 4)
    plan["chain_attn_bda_bwd_bf16_16384x8192"] = (bda_bwd(c5, "attn_g", "bf16", 0.1, 5001, False),
                                                  lambda n: n * 8192 * 4 + 8192 * 4)
    plan["erf_gelu_fwd_bf16_16384x32768"] = (gelu_fwd(True), lambda n: n * 32768 * 4 + 32768 * 2)
    plan["erf_gelu_bwd_bf16_16384x32768"] = (gelu_bwd(True), lambda n: n * 32768 * 6 + 32768 * 6)

    for wname in ("add_ln_bf16_16384x8192", "add_ln_bf16_8192x16384", "add_ln_bf16_2048x65536"):
        tag = wname[len("add_ln_"):]
        H = host[(wname, "gamma")].shape[0]
        kb = 128 * 2.0**-24  # the derived bound of the fp32 row sums, times mag

        def ln_fwd(r0, r1, w=wname):
            h, y, y64, mag, _, _ = oracle.add_layer_norm_fwd("bf16", rows(w, "x", r0, r1), rows(w, "residual", r0, r1),
                                                             "bf16", vec(w, "gamma"), vec(w, "beta"), 1e-5, True)
            return {"h": ("exact", h), "y": ("bounded", y, y64, kb * mag)}

        def ln_bwd(r0, r1, w=wname):
            h, _, _, _, _, _ = oracle.add_layer_norm_fwd("bf16", rows(w, "x", r0, r1), rows(w, "residual", r0, r1),
                                                         "bf16", vec(w, "gamma"), vec(w, "beta"), 1e-5, True)
            dx, dx64, mag, _, _, _ = oracle.add_layer_norm_bwd("bf16", rows(w, "dy", r0, r1), h, vec(w, "gamma"), 1e-5,
                                                               True, dh_in=rows(w, "dh_in", r0, r1), want_dres=False)
            return {"dx": ("bounded", dx, dx64, kb * mag)}

        def ln_fwd32(r0, r1, w=wname):
            h, y, _, _ = oracle32.add_layer_norm_fwd("bf16", rows(w, "x", r0, r1), rows(w, "residual", r0, r1), "bf16",
                                                     vec(w, "gamma"), vec(w, "beta"), 1e-5, True)
            return {"h": h, "y": y}

        def ln_bwd32(r0, r1, w=wname):
            h = ln_fwd32(r0, r1, w)["h"]
            dx, _, _, _ = oracle32.add_layer_norm_bwd("bf16", rows(w, "dy", r0, r1), h, vec(w, "gamma"), 1e-5, True,
                                                      dh_in=rows(w, "dh_in", r0, r1), want_dres=False)
            return {"dx": dx}

        plan[f"add_ln_fwd_{tag}"] = (ln_fwd, lambda n, H=H: n * H * 8 + H * 4 + n * 8)
        plan[f"add_ln_bwd_{tag}"] = (ln_bwd, lambda n, H=H: n * H * 8 + H * 2 + n * 8 + H * 8)
        plan32[f"add_ln_fwd_{tag}"] = ln_fwd32
        plan32[f"add_ln_bwd_{tag}"] = ln_bwd32

    c7 = "wsrelu_bf16_8192x14336"

    def srelu_fwd(r0, r1):
        o, o64 = oracle.weighted_squared_relu_fwd("bf16", rows(c7, "x", r0, r1), rows(c7, "weights", r0, r1), "f32")
        return {"out": ("elem", o, o64, None)}

    def srelu_bwd(r0, r1):
        d, d64, dw = oracle.weighted_squared_relu_bwd("bf16", rows(c7, "g", r0, r1), rows(c7, "x", r0, r1),
                                                      rows(c7, "weights", r0, r1), "f32")
        return {"dx": ("elem", d, d64, None), "dweights": ("rowsum", dw)}

    plan["weighted_squared_relu_fwd_bf16_8192x14336"] = (srelu_fwd, lambda n: n * 14336 * 4 + n * 4)
    plan["weighted_squared_relu_bwd_bf16_8192x14336"] = (srelu_bwd, lambda n: n * 14336 * 6 + n * 8)
    plan32["weighted_squared_relu_fwd_bf16_8192x14336"] = lambda r0, r1: {"out": oracle32.weighted_squared_relu_fwd(
        "bf16", rows(c7, "x", r0, r1), rows(c7, "weights", r0, r1), "f32")}
    plan32["weighted_squared_relu_bwd_bf16_8192x14336"] = lambda r0, r1: {"dx": oracle32.weighted_squared_relu_bwd(
        "bf16", rows(c7, "g", r0, r1), rows(c7, "x", r0, r1), rows(c7, "weights", r0, r1), "f32")[0]}
    del np
    rows_of = {"bda_": c2, "swiglu": c3, "weighted_swiglu": c3, "geglu": c4, "chain_": c5, "erf_gelu": c5,
               "weighted_squared": "wsrelu_bf16_8192x14336"}
    out = {}
    for name, (f, nb) in plan.items():
        if name.startswith("add_ln_"):
            w = "add_ln_" + name.split("_", 3)[3]
        else:
            w = next(v for k, v in rows_of.items() if name.startswith(k))
        first = next(t for (wn, _), t in host.items() if wn == w and t.dim() == 2)
        out[name] = (f, nb, first.shape[0], plan32[name])
    return out


def parity_stats(expected, got):
    """Per output of one op: the comparator's statistics of the GPU rows against
    the oracle's (same rows, same inputs)."""
    import numpy as np

    from oracle.tolerances import assert_reduction_close, compare

    res = {}
    for name, exp in expected.items():
        k = got[name]
        kind = exp[0]
        if kind == "exact":
            eq = k.view(np.uint32 if k.dtype == np.float32 else np.uint16) == \
                exp[1].view(np.uint32 if exp[1].dtype == np.float32 else np.uint16)
            res[name] = {"n": int(eq.size), "fail": int((~eq).sum()), "kind": "bit-exact"}
        elif kind == "rowsum":
            try:
                r = assert_reduction_close(k, exp[1], name)
                res[name] = {"n": r["n"], "fail": 0, "max_rel_to_rms": round(r["max_rel_to_rms"], 8),
                             "kind": "fp32 row sum, 1e-3"}
            except AssertionError as e:
                res[name] = {"n": int(exp[1].size), "fail": -1, "error": str(e)[:200]}
        elif kind == "bounded":
            from oracle.tolerances import values, ulp

            dt = "bf16"
            kv, ov = values(k, dt), values(exp[1], dt)
            with np.errstate(invalid="ignore"):
                ok = (np.abs(kv - ov) <= ulp(ov, dt)) | (np.abs(kv - exp[2]) <= exp[3] + ulp(exp[2], dt))
            ok |= k.view(np.uint16) == exp[1].view(np.uint16)
            res[name] = {"n": int(ok.size), "fail": int((~ok).sum()), "kind": "1 ulp or derived row-sum bound"}
        else:
            dt = "f32" if k.dtype == np.float32 else "bf16"
            _, st = compare(k, exp[1], exp[2], exp[3], dt)
            st["kind"] = "1e-6 rel + 1e-6" if dt == "f32" else "1 ulp (bf16)"
            res[name] = {key: (round(v, 6) if isinstance(v, float) else v) for key, v in st.items()}
    return res


def oracle32_stats(exp32, got):
    """Secondary statistic per output: the GPU's storage against oracle32's
    (the formulas in binary32): elements bit-equal, and the largest distance in
    units of the last place of the storage type."""
    import numpy as np

    res = {}
    for name, e in exp32.items():
        if name not in got:
            continue
        k = got[name]
        if k.dtype == np.float32:
            ki, ei = k.view(np.int32).astype(np.int64), e.view(np.int32).astype(np.int64)
            ki = np.where(ki < 0, -(ki & 0x7FFFFFFF), ki)
            ei = np.where(ei < 0, -(ei & 0x7FFFFFFF), ei)
        else:
            ki, ei = k.view(np.int16).astype(np.int64), e.view(np.int16).astype(np.int64)
            ki = np.where(ki < 0, -(ki & 0x7FFF), ki)
            ei = np.where(ei < 0, -(ei & 0x7FFF), ei)
        d = np.abs(ki - ei)
        res[name] = {"n": int(d.size), "bit_equal": int((d == 0).sum()), "max_ulp": int(d.max()) if d.size else 0}
    return res


def cpu_baseline(host, gpu_rows, seconds, max_rows=512, max_threads=16):
    """The oracle (C, fp64) on the first rows of every op's inputs, as the same
    algorithmic bytes per second: on one pinned core, and on a pool of threads
    over row chunks (the oracle's calls release the interpreter lock); the
    single-core outputs are compared with the GPU's rows. oracle32 (the same
    formulas in binary32) is timed the same way on the same rows, and the GPU's
    rows are compared with it as a secondary statistic."""
    from oracle.tolerances import to_storage

    plan = oracle_plan(host)
    names = [n for n in plan if n in gpu_rows]
    info = cpu_info()
    threads = max(1, min(max_threads, info["available"]))
    try:
        old_aff = os.sched_getaffinity(0)
        os.sched_setaffinity(0, {min(old_aff)})
    except (AttributeError, OSError):
        old_aff = None
    try:
        t0 = time.perf_counter()
        for n in names:
            plan[n][0](0, 2)
        probe = time.perf_counter() - t0
        n1 = max(2, min(max_rows, int(2 * seconds / max(probe, 1e-6))))
        tot_b, tot_s, per, parity = 0, 0.0, {}, {}
        tot_s32, per32 = 0.0, {}
        for name in names:
            f, nb, _, f32 = plan[name]
            t0 = time.perf_counter()
            exp = f(0, n1)
            dt = time.perf_counter() - t0
            tot_b += nb(n1)
            tot_s += dt
            per[name] = round(nb(n1) / dt / 1e9, 4)
            t0 = time.perf_counter()
            exp32 = f32(0, n1)
            dt32 = time.perf_counter() - t0
            tot_s32 += dt32
            per32[name] = round(nb(n1) / dt32 / 1e9, 4)
            got = {k: (to_storage(v[:n1]) if v.dim() == 2 else v[:n1].double().numpy()) for k, v in gpu_rows[name].items()}
            parity[name] = parity_stats(exp, got)
            parity[name]["vs_oracle32"] = oracle32_stats(exp32, got)
        single = {"value": round(tot_b / tot_s / 1e9, 4), "cores": 1, "rows": n1, "seconds": round(tot_s, 2),
                  "per_op_gbs": per}
        single32 = {"value": round(tot_b / tot_s32 / 1e9, 4), "cores": 1, "rows": n1, "seconds": round(tot_s32, 2),
                    "per_op_gbs": per32}
    finally:
        if old_aff is not None:
            os.sched_setaffinity(0, old_aff)
    # the thread pool: row chunks of a larger sample (the oracle is row-local;
    # the dropout rows carry their global row index), same ops
    want = max(threads * 2, n1 * threads)
    tot_b, tot_s, tot_s32, rows_used = 0, 0.0, 0.0, {}
    with ThreadPoolExecutor(threads) as ex:
        for name in names:
            f, nb, T, f32 = plan[name]
            nt = min(want, T)
            step = (nt + threads - 1) // threads
            chunks = [(r0, min(nt, r0 + step)) for r0 in range(0, nt, step)]
            t0 = time.perf_counter()
            list(ex.map(lambda c: f(*c), chunks))
            tot_s += time.perf_counter() - t0
            t0 = time.perf_counter()
            list(ex.map(lambda c: f32(*c), chunks))
            tot_s32 += time.perf_counter() - t0
            tot_b += nb(nt)
            rows_used[name] = nt
    nt = max(rows_used.values())
    pool = {"value": round(tot_b / tot_s / 1e9, 4), "cores": threads, "rows": rows_used, "seconds": round(tot_s, 2)}
    pool32 = {"value": round(tot_b / tot_s32 / 1e9, 4), "cores": threads, "seconds": round(tot_s32, 2)}
    return {"value": pool["value"], "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"first min({want}, T) rows of every op's inputs (same ops, shapes and seeds as the GPU "
                      f"step and next rows), fp64 C oracle over {threads} threads in row chunks, {pool['seconds']} s; "
                      f"single pinned core: first {n1} rows, {single['value']} GB/s",
            "cpu": info, "single_core": single, "thread_pool": pool,
            "oracle32": {"note": "the same formulas in binary32 (plain fp32 scalar C), same rows",
                         "single_core": single32, "thread_pool": pool32}}, parity


# ------------------------------------------------------------------ main

def device_info(dev):
    """Architecture and compute-unit count of the measured device."""
    import torch

    p = torch.cuda.get_device_properties(dev)
    return {"arch": p.gcnArchName.split(":")[0], "compute_units": p.multi_processor_count}


def capture_steps(ops, nsteps, stream):
    """One HIP graph per step j (call index j of every op)."""
    import torch

    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        for op in ops:
            op.call(0)
    stream.wait_stream(side)
    torch.cuda.synchronize()
    graphs = []
    for j in range(nsteps):
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for op in ops:
                op.call(j)
        graphs.append(gr)
    return graphs


def refresh(ops):
    for op in ops:
        if op.refresh:
            op.refresh()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py: runs on one GPU only (asked for --gpus {args.gpus}); "
              "the fused epilogues are per-token and would shard by rows with a dbias all-reduce, "
              "which is not built here.", file=sys.stderr)
        sys.exit(2)
    import torch

    if not torch.cuda.is_available():
        print("bench.py: no GPU visible", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    K, W = args.steps, args.warmup
    if args.copy_calibration:
        a = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        del a, b
        torch.cuda.empty_cache()
    t_setup = time.perf_counter()
    log("building inputs")
    ops, extra, host = build_ops(dev, max(K, W, 1))
    L = stream_lib()
    torch.cuda.synchronize()
    setup_s = time.perf_counter() - t_setup
    stream = torch.cuda.current_stream(dev)

    # -- per-op durations: eager launches, HIP events around every op
    log(f"inputs ready in {setup_s:.1f} s; timing the step")
    for s in range(W):
        for op in ops:
            op.call(s)
    refresh(ops)
    torch.cuda.synchronize()
    ev = [events(len(ops)) for _ in range(K)]
    step0, step1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    step0.record(stream)
    for s in range(K):
        for op, (e0, e1) in zip(ops, ev[s]):
            e0.record(stream)
            op.call(s)
            e1.record(stream)
    step1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms_per_step_eager = step0.elapsed_time(step1) / K
    for s in range(K):
        for op, (e0, e1) in zip(ops, ev[s]):
            op.ms.append(e0.elapsed_time(e1))
    step_bytes = sum(op.nbytes for op in ops)
    launch, ms_per_step = "eager", ms_per_step_eager
    if not args.eager:
        # the step captured into one HIP graph per timed step (every entry
        # point issues only kernel launches, so it is capturable) and replayed:
        # the same kernels and bytes, without the per-launch host and queue gaps
        graphs = capture_steps(ops, K, stream)
        for j in range(min(W, K)):
            graphs[j].replay()
        refresh(ops)
        torch.cuda.synchronize()
        wall0 = time.perf_counter()
        step0.record(stream)
        for gr in graphs:
            gr.replay()
        step1.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - wall0
        ms_per_step = step0.elapsed_time(step1) / K
        launch = "hip_graph"
        del graphs
    value = step_bytes / (ms_per_step * 1e-3) / 1e9

    # -- the ops beyond the step, after it, in a loop of their own
    log(f"step {ms_per_step:.4f} ms ({launch}); timing the next rows")
    for _ in range(W):
        for op in extra:
            op.call(0)
    xev = [events(len(extra)) for _ in range(K)]
    for s in range(K):
        for op, (e0, e1) in zip(extra, xev[s]):
            e0.record(stream)
            op.call(s)
            e1.record(stream)
    torch.cuda.synchronize()
    for s in range(K):
        for op, (e0, e1) in zip(extra, xev[s]):
            op.ms.append(e0.elapsed_time(e1))

    # -- C1 cold and warm
    log("timing the fp32 GeLU at [512, 4096], cold and warm")
    c1 = c1_bench(dev, L, stream, not args.no_ceiling)

    # -- the streaming ceiling of every op (writes junk into the op's outputs)
    ceil, tables = {}, {}
    if not args.no_ceiling:
        for op in ops + extra:
            tables[op.name] = {} if args.ceiling_table else None
            ceil[op.name] = ceiling(op, L, stream, tables[op.name])
            log(f"ceiling {op.name}: {ceil[op.name]}")
        if args.ceiling_table:
            with open(args.ceiling_table, "w") as fh:
                json.dump(tables, fh)

    # -- the outputs of call 0 of every op on fresh inputs, for the parity statistics
    gpu_rows = {}
    nrow = 512
    if not args.no_cpu_baseline:
        refresh(ops)
        for op in ops + extra:
            op.call(0)
            torch.cuda.synchronize()
            gpu_rows[op.name] = {k: v[:nrow].cpu() for k, v in op.outputs.items()}

    def stats(group):
        res = {}
        for op in group:
            avg = sum(op.ms) / len(op.ms)
            gbs = op.nbytes / (avg * 1e-3) / 1e9
            r = {"us": round(avg * 1e3, 2), "bytes": op.nbytes, "gbs": round(gbs, 1),
                 "frac_peak": round(gbs / PEAK_HBM_GBS, 4), "kernels": op.kernels}
            if op.name in ceil:
                c = ceil[op.name]
                r["ceiling"] = c
                r["frac_ceiling"] = round(c["us"] / (avg * 1e3), 4)
            res[op.name] = r
        return res

    per_op, next_rows = stats(ops), stats(extra)
    dom = max(ops, key=lambda o: sum(o.ms))
    dom_avg = sum(dom.ms) / len(dom.ms)
    achieved = dom.nbytes / (dom_avg * 1e-3) / 1e9
    traffic = measured_traffic() if dom.name == "chain_gelu_bwd_bf16_16384x32768" else None
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": PEAK_HBM_GBS, "unit": "GB/s",
                "frac": round(achieved / PEAK_HBM_GBS, 4), "traffic": traffic,
                "kernel": dom.name, "launches": dom.kernels, "algorithmic_bytes_per_launch": dom.nbytes,
                "avg_us": round(dom_avg * 1e3, 2)}
    if dom.name in ceil:
        roofline["frac_ceiling"] = per_op[dom.name]["frac_ceiling"]
        roofline["ceiling_gbs"] = ceil[dom.name]["gbs"]
    cpu = parity = None
    if not args.no_cpu_baseline:
        log("CPU baseline and parity statistics")
        cpu, parity = cpu_baseline(host, gpu_rows, args.cpu_seconds)
    config = {"workload": WORKLOAD, "storage": "bf16 (fp32 residual in the 8192x4096 dropout-add)",
              "arithmetic": "f32 in registers, each output rounded once",
              "step_bytes": step_bytes, "frac_peak": round(value / PEAK_HBM_GBS, 4), "launch": launch,
              "ms_per_step_eager": round(ms_per_step_eager, 4), "device": device_info(dev)}
    if ceil:
        step_ceiling_us = sum(ceil[op.name]["us"] for op in ops)
        config["step_ceiling_ms"] = round(step_ceiling_us / 1e3, 4)
        config["frac_ceiling"] = round(step_ceiling_us / 1e3 / ms_per_step, 4)
    line = {
        "metric": "achieved HBM GB/s and % of MI355X peak per fused op (fwd+bwd), 1 GPU",
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": W,
        "ms_per_step": round(ms_per_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic (seeded numpy normal/uniform, cast to bf16; resident in HBM before timing)",
        "config": config,
        "per_op": per_op,
        "next_rows": next_rows,
        "c1": c1,
        "roofline": roofline,
        "cpu_baseline": cpu,
        "parity": parity,
        "wall_s": round(wall, 3),
        "setup_s": round(setup_s, 1),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
