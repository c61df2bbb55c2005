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
OK, NULL, SHAPE, DTYPE, ALIGN, ALIAS, PROB, WORKSPACE = range(8)
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
    for code in range(9):
        assert L.mb_status_string(code).startswith(b"MB_")


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
