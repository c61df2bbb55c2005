"""The C-ABI library without a GPU: it loads, exports every function that
include/mb.h declares, and its host-side validation rejects bad arguments
before any HIP call (fabricated pointer values are never dereferenced)."""
import ctypes
import os
import re

import pytest

import transformer_elementwise_epilogues_amd as mb

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "mb.h")
OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, PROB, WORKSPACE, HIP, SCRATCH = range(10)
F32, F16, BF16 = 0, 1, 2


def declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(mb_[a-z0-9_]+)\s*\(", text)))


def test_header_declares_the_entry_points():
    names = declared()
    for n in ["mb_bias_gelu_fwd", "mb_bias_gelu_bwd", "mb_bias_dropout_add_train", "mb_bias_dropout_add_infer",
              "mb_bias_swiglu_fwd", "mb_bias_swiglu_bwd", "mb_bias_geglu_fwd", "mb_bias_geglu_bwd",
              "mb_dropout_mask", "mb_status_string", "mb_abi_version"]:
        assert n in names


def test_library_exports_every_declared_symbol():
    L = ctypes.CDLL(mb.LIB_PATH)
    missing = [n for n in declared() if not hasattr(L, n)]
    assert not missing, missing


def test_version_and_status_strings():
    assert mb.abi_version() == 1
    L = mb.lib()
    for code in range(10):
        assert L.mb_status_string(code).startswith(b"MB_")
    assert b"scratch" in L.mb_status_string(SCRATCH)


# Fake, 256-byte aligned "device" addresses: validation never touches them.
A, B, C, D, E = (0x10000000 * k for k in range(1, 6))


def L():
    return mb.lib()


def test_gelu_fwd_validation():
    f = L().mb_bias_gelu_fwd
    assert f(A, None, B, 4, 63, BF16, None) == SHAPE       # 63 bf16 is not whole 16-byte vectors
    assert f(A, None, B, 4, 6, F32, None) == SHAPE
    assert f(A, None, B, -1, 64, BF16, None) == SHAPE
    assert f(A, None, B, 4, 0, BF16, None) == SHAPE
    assert f(A, None, B, 4, 64, 7, None) == DTYPE
    assert f(None, None, B, 4, 64, BF16, None) == NULL
    assert f(A + 2, None, B, 4, 64, BF16, None) == ALIGN
    assert f(A, C + 8, B, 4, 64, BF16, None) == ALIGN
    assert f(A, None, A + 16, 4, 64, BF16, None) == ALIAS  # partial overlap
    assert f(A, None, B, 0, 64, BF16, None) == OK          # empty: nothing enqueued
    assert f(A, None, B, 2**62, 2**20, BF16, None) == SHAPE  # byte size overflows


def test_gelu_bwd_validation():
    f = L().mb_bias_gelu_bwd
    ws = L().mb_bias_gelu_bwd_workspace(1024, 4096, BF16, 1)
    assert ws > 0 and L().mb_bias_gelu_bwd_workspace(1024, 4096, BF16, 0) == 0
    assert L().mb_bias_gelu_bwd_workspace(0, 4096, BF16, 1) == 0
    assert f(A, B, None, C, D, None, 0, 1024, 4096, BF16, None) == WORKSPACE
    assert f(A, B, None, C, D, E, ws - 1, 1024, 4096, BF16, None) == WORKSPACE
    assert f(A, B, None, C, D + 2, E, ws, 1024, 4096, BF16, None) == ALIGN
    assert f(A, B, None, C, D, E + 4, ws, 1024, 4096, BF16, None) == ALIGN
    assert f(A, B, None, C, C + 64, E, ws, 1024, 4096, BF16, None) == ALIAS   # dbias inside dgrad
    assert f(A, B, None, C, D, C, ws, 1024, 4096, BF16, None) == ALIAS        # ws over dgrad
    assert f(A, B, None, B + 16, None, None, 0, 1024, 4096, BF16, None) == ALIAS
    # the exact form has its own launch shape and workspace query
    wse = L().mb_bias_gelu_erf_bwd_workspace(1024, 4096, BF16, 1)
    assert wse > 0 and L().mb_bias_gelu_erf_bwd_workspace(1024, 4096, BF16, 0) == 0
    fe = L().mb_bias_gelu_erf_bwd
    assert fe(A, B, None, C, D, E, wse - 1, 1024, 4096, BF16, None) == WORKSPACE
    assert fe(A, B, None, C, D, None, 0, 1024, 4096, BF16, None) == WORKSPACE


def test_bda_validation():
    tr, inf = L().mb_bias_dropout_add_train, L().mb_bias_dropout_add_infer
    for p in (-0.5, 1.01, float("nan"), float("inf")):
        assert tr(A, None, B, F32, C, 8, 64, BF16, p, 1, 0, None) == PROB
    assert tr(A, None, B, F16, C, 8, 64, BF16, 0.1, 1, 0, None) == DTYPE   # residual must be dt or fp32
    assert inf(A, None, B, F32, A, 0, 64, BF16, None) == OK                 # in place, empty
    assert inf(A, None, B, BF16, B, 0, 64, BF16, None) == OK                # in place on residual
    assert inf(A, None, B, F32, B, 8, 64, BF16, None) == ALIAS              # fp32 residual is not out's size
    assert inf(A, None, None, F32, C, 8, 64, BF16, None) == NULL
    assert inf(A, None, B + 8, F32, C, 8, 64, BF16, None) == ALIGN


def test_mask_validation():
    f = L().mb_dropout_mask
    assert f(A, 4, 6, 0.1, 1, 0, None) == SHAPE
    assert f(A, 4, 8, 2.0, 1, 0, None) == PROB
    assert f(None, 4, 8, 0.1, 1, 0, None) == NULL
    assert f(None, 0, 8, 0.1, 1, 0, None) == OK


def test_glu_validation():
    fw, bw = L().mb_bias_swiglu_fwd, L().mb_bias_swiglu_bwd
    assert fw(A, None, None, BF16, B, 8, 60, BF16, None) == SHAPE
    assert fw(A, None, C, F16, B, 8, 64, BF16, None) == DTYPE
    assert fw(A, None, C + 1, BF16, B, 8, 64, BF16, None) == ALIGN
    assert fw(A, None, None, BF16, A + 512, 8, 64, BF16, None) == ALIAS   # out inside in
    assert fw(A, None, None, BF16, A, 8, 64, BF16, None) == ALIAS         # no in-place forward
    ws = L().mb_bias_glu_bwd_workspace(64, 512, BF16, 1, 1)
    assert ws > L().mb_bias_glu_bwd_workspace(64, 512, BF16, 1, 0) > 0
    assert bw(A, B, None, None, BF16, C, None, D, E, ws, 64, 512, BF16, None) == NULL  # dweights needs weights
    assert bw(A, B, None, E, BF16, C, D, D + 4096 * 4, None, 0, 64, 512, BF16, None) == WORKSPACE
    assert bw(A, B, None, None, BF16, A, None, None, None, 0, 64, 512, BF16, None) == ALIAS  # din over g
    assert bw(A, B, None, None, BF16, B, None, None, None, 0, 0, 512, BF16, None) == OK      # in place, empty


def test_layer_norm_validation():
    fw, bw, wsf = L().mb_add_layer_norm_fwd, L().mb_add_layer_norm_bwd, L().mb_add_layer_norm_bwd_workspace
    # (x, residual, residual_dt, gamma, beta, eps, zero_centered, h_out, y, mean, rstd, T, H, dt, stream)
    assert fw(A, B, BF16, C, None, 1e-5, 0, None, D, None, None, 4, 60, BF16, None) == SHAPE   # not whole vectors
    assert fw(A, B, BF16, C, None, 1e-5, 0, None, D, None, None, 0, 65536, BF16, None) == OK
    assert fw(A, B, BF16, C, None, 1e-5, 0, None, D, None, None, 4, 65536 + 8, BF16, None) == SHAPE  # too wide
    assert fw(A, B, F32, C, None, 1e-5, 0, None, D, None, None, 0, 32768, BF16, None) == OK
    assert fw(A, B, F32, C, None, 1e-5, 0, None, D, None, None, 4, 32768 + 4, BF16, None) == SHAPE
    assert fw(A, B, F32, C, None, 1e-5, 0, None, D, None, None, 0, 36, BF16, None) == OK       # 4-element pieces
    assert fw(A, B, F32, C, None, 1e-5, 0, None, D, None, None, 4, 32772, F32, None) == SHAPE
    assert fw(A, B, F16, C, None, 1e-5, 0, None, D, None, None, 4, 64, BF16, None) == DTYPE     # residual dt or fp32
    for eps in (-1.0, float("nan"), float("inf")):
        assert fw(A, B, BF16, C, None, eps, 0, None, D, None, None, 4, 64, BF16, None) == PROB
    assert fw(A, B, BF16, None, None, 1e-5, 0, None, D, None, None, 4, 64, BF16, None) == NULL  # gamma required
    assert fw(A, B, BF16, C, None, 1e-5, 0, None, D, E, None, 4, 64, BF16, None) == NULL        # mean without rstd
    assert fw(A + 8, B, BF16, C, None, 1e-5, 0, None, D, None, None, 4, 64, BF16, None) == ALIGN
    assert fw(A, B, BF16, C, None, 1e-5, 0, D, D, None, None, 4, 64, BF16, None) == ALIAS       # h_out == y
    assert fw(A, B, BF16, C, None, 1e-5, 0, None, C, None, None, 4, 64, BF16, None) == ALIAS    # y over gamma
    assert fw(A, B, BF16, C, None, 1e-5, 0, A, B, None, None, 0, 64, BF16, None) == OK          # h into x, y into r
    assert fw(A, B, F32, C, None, 1e-5, 0, None, B, None, None, 4, 64, BF16, None) == ALIAS     # y over fp32 residual
    # backward (dy, h, gamma, mean, rstd, zc, dh_in, rdt, dx, dres, dgamma, dbeta, ws, ws_bytes, T, H, dt, stream)
    ws = wsf(1024, 8192, BF16, BF16, 1)
    assert ws > 0 and wsf(1024, 8192, BF16, BF16, 0) == 0 and wsf(0, 8192, BF16, BF16, 1) == 0
    assert wsf(1024, 65536, BF16, BF16, 1) > 0
    # rows of more than 2048 vectors keep row sums even without parameter
    # gradients: a team of ceil(vectors / 1024) blocks exchanges one pair of
    # fp32 partial sums per row and member, plus a row flag (the in-place
    # wide-row kernels need less: 2 fp32 sums per row); rows of 1025-2048
    # vectors need none
    team = lambda T, members: -(-T * (members * 8 + 4) // 256) * 256
    assert wsf(1024, 65536, BF16, BF16, 0) == team(1024, 8) and wsf(1000, 32768, BF16, BF16, 0) == team(1000, 4)
    assert wsf(1024, 16384, BF16, F32, 0) == team(1024, 4) and wsf(1024, 16384, F32, F32, 0) == team(1024, 4)
    assert wsf(1000, 16384, BF16, BF16, 0) == 0 and wsf(1024, 8192, BF16, F32, 0) == 0
    assert wsf(1024, 8200, BF16, BF16, 1) > 0
    assert bw(A, B, C, D, E, 0, None, BF16, 0x60000000, None, None, None, None, 0, 1024, 65536, BF16,
              None) == WORKSPACE
    assert bw(A, B, C, D, E, 0, None, BF16, 0x60000000, None, 0x70000000, None, None, 0, 1024, 8192, BF16,
              None) == WORKSPACE
    assert bw(A, B, C, D, None, 0, None, BF16, 0x60000000, None, None, None, None, 0, 1024, 8192, BF16,
              None) == NULL
    assert bw(A, B, C, D, E, 0, None, BF16, A + 16, None, None, None, None, 0, 1024, 8192, BF16, None) == ALIAS
    assert bw(A, B, C, D, E, 0, None, BF16, A, B, None, None, None, 0, 0, 8192, BF16, None) == OK  # dx = dy, dres = h
    # (bf16 beside an fp32 residual: 4096 vectors of 4, a two-pass row that needs its row-sum workspace)
    assert bw(A, B, C, D, E, 0, None, F32, A, B, None, None, 0x60000000, 4096, 4, 16384, BF16, None) == ALIAS


def test_squared_relu_validation():
    fw, bw, wsf = (L().mb_weighted_squared_relu_fwd, L().mb_weighted_squared_relu_bwd,
                   L().mb_weighted_squared_relu_bwd_workspace)
    assert fw(A, None, F32, B, 4, 60, BF16, None) == SHAPE
    assert fw(A, C, 7, B, 4, 64, BF16, None) == DTYPE
    assert fw(A, C + 2, F32, B, 4, 64, BF16, None) == ALIGN       # fp32 weights need 4-byte alignment
    assert fw(A, None, F32, A + 16, 4, 64, BF16, None) == ALIAS
    assert fw(A, None, F32, A, 0, 64, BF16, None) == OK           # in place, empty
    ws = wsf(64, 512, BF16, 1)
    assert ws > 0 and wsf(64, 512, BF16, 0) == 0
    assert bw(A, B, None, F32, C, D, E, ws, 64, 512, BF16, None) == NULL        # dweights needs weights
    assert bw(A, B, E, F32, C, D, None, 0, 64, 512, BF16, None) == WORKSPACE
    assert bw(A, B, None, F32, A, None, None, 0, 0, 512, BF16, None) == OK      # dx over g, empty
    assert bw(A, B, None, F32, A + 16, None, None, 0, 4, 512, BF16, None) == ALIAS


def test_gelu_bwd_noalloc_validation():
    """The entry point without a workspace: the same checks as mb_bias_gelu_bwd,
    and rows too wide for its static scratch refused before any HIP call."""
    f = L().mb_bias_gelu_bwd_noalloc
    assert f(A, B, None, C, D, 4, 63, BF16, None) == SHAPE
    assert f(A, B, None, C, D, 4, 64, 7, None) == DTYPE
    assert f(None, B, None, C, D, 4, 64, BF16, None) == NULL
    assert f(A, B, None, C, D + 2, 4, 64, BF16, None) == ALIGN
    assert f(A, B, None, C, C + 64, 4, 64, BF16, None) == ALIAS      # dbias inside dgrad
    assert f(A, B, None, B + 16, None, 4, 64, BF16, None) == ALIAS   # dgrad partly over y
    wide = (16 << 20) // 4 + 8                                      # one fp32 row exceeds 16 MiB
    assert f(A, B, None, C, D, 1, wide, BF16, None) == SCRATCH
    assert f(A, B, None, C, D, 0, wide, BF16, None) == SCRATCH
