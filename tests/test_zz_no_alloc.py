"""mb_bias_gelu_bwd_noalloc through the C ABI against mb_bias_gelu_bwd.

The no-allocation entry point keeps the bias gradient's partial rows in the
library's static device scratch. Two calls in a row, the second with a
smaller input (the scratch still holds the first call's larger partials),
must each give dgrad bit for bit equal to the workspace entry point's and
dbias within the reduction tolerance of it and of the oracle."""
import ctypes

import numpy as np
import pytest
import torch

import oracle
import transformer_elementwise_epilogues_amd as mb
from transformer_elementwise_epilogues_amd import synthetic
from tolerances import assert_reduction_close, to_storage

pytestmark = pytest.mark.gpu
DEV = torch.device("cuda:0")
TD = {"f32": torch.float32, "bf16": torch.bfloat16, "f16": torch.float16}
SCRATCH, SCRATCH_ERR = 16 << 20, 9


def noalloc(g, y, bias, dgrad, dbias):
    T, H = y.shape
    return mb.lib().mb_bias_gelu_bwd_noalloc(
        ctypes.c_void_p(g.data_ptr()), ctypes.c_void_p(y.data_ptr()),
        None if bias is None else ctypes.c_void_p(bias.data_ptr()), ctypes.c_void_p(dgrad.data_ptr()),
        None if dbias is None else ctypes.c_void_p(dbias.data_ptr()), T, H, mb.DTYPES[y.dtype],
        ctypes.c_void_p(torch.cuda.current_stream(DEV).cuda_stream))


def run_pair(dt, T, H, seed, with_oracle):
    y = synthetic.draw(seed, (T, H), "normal", 1.0, dt)
    g = synthetic.draw(seed + 1, (T, H), "normal", 1.0, dt)
    b = synthetic.draw(seed + 2, (H,), "normal", 0.02, dt)
    yd, gd, bd = y.to(DEV), g.to(DEV), b.to(DEV)
    dg_ref, db_ref = mb.mb_bias_gelu_bwd(gd, yd, bd)
    dg = torch.full_like(yd, float("nan"))
    db = torch.full((H,), float("nan"), dtype=torch.float32, device=DEV)
    print(f"[noalloc] {dt} T={T} H={H}", flush=True)
    assert noalloc(gd, yd, bd, dg, db) == 0
    torch.cuda.synchronize()
    assert torch.equal(dg.view(torch.int16 if dt != "f32" else torch.int32),
                       dg_ref.view(torch.int16 if dt != "f32" else torch.int32)), "dgrad differs"
    assert_reduction_close(db.cpu().numpy(), db_ref.cpu().numpy().astype(np.float64), f"dbias vs workspace {dt}")
    if with_oracle:
        _, _, _, db64 = oracle.bias_gelu_bwd(dt, to_storage(g), to_storage(y), to_storage(b))
        assert_reduction_close(db.cpu().numpy(), db64, f"dbias vs oracle {dt}")
    return db


def test_noalloc_two_calls_second_smaller():
    # first: 64 column strips and more row groups than the scratch allows
    # (capped at 128 partial rows); second: 3 strips, the last one ragged
    run_pair("bf16", 4096, 32768, 71, with_oracle=False)
    run_pair("bf16", 300, 1040, 81, with_oracle=True)


def test_noalloc_fp32_and_repeat_is_bit_identical():
    a = run_pair("f32", 512, 4096, 91, with_oracle=True)
    b = run_pair("f32", 512, 4096, 91, with_oracle=False)
    assert torch.equal(a, b)


def test_noalloc_without_dbias_and_empty():
    y = synthetic.draw(5, (64, 512), "normal", 1.0, "bf16").to(DEV)
    g = synthetic.draw(6, (64, 512), "normal", 1.0, "bf16").to(DEV)
    dg = torch.empty_like(y)
    assert noalloc(g, y, None, dg, None) == 0
    ref, _ = mb.mb_bias_gelu_bwd(g, y, dbias=False)
    e = torch.empty((0, 512), dtype=torch.bfloat16, device=DEV)
    db = torch.full((512,), 7.0, dtype=torch.float32, device=DEV)
    assert noalloc(e, e, None, e, db) == 0  # empty: the bias gradient is zeros
    torch.cuda.synchronize()
    assert torch.equal(dg.view(torch.int16), ref.view(torch.int16))
    assert torch.count_nonzero(db).item() == 0


def test_noalloc_refuses_rows_beyond_the_scratch():
    H = SCRATCH // 4 + 8  # one fp32 partial row no longer fits
    y = torch.zeros((1, H), dtype=torch.bfloat16, device=DEV)
    db = torch.zeros(H, dtype=torch.float32, device=DEV)
    assert noalloc(y, y, None, torch.empty_like(y), db) == SCRATCH_ERR
    assert b"scratch" in mb.lib().mb_status_string(SCRATCH_ERR)
    with pytest.raises(mb.MBError, match="MB_ERR_SCRATCH"):
        mb.mb_bias_gelu_bwd_noalloc(y, y, dbias=db)
