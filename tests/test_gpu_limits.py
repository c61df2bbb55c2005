"""The size limits of the ABI on the GPU, against the oracle on sampled rows
or columns:

- a dropout mask of 2^34 + 2^20 elements (2 GiB of bits): element indices
  past 2^34 use the high word of the Philox counter's element half;
- a dropout-add over 2^32 + 2^18 elements (8.6 GB per tensor): element
  indices and byte offsets past 32 bits in the fused kernel;
- GeLU forward and backward at the widest hidden size the tiling accepts
  (65535 column strips of 64 vectors: 33 553 920 bf16 per row), and one
  vector more is refused;
- GeLU backward over 2^24 rows of 64 columns (row groups capped, long row
  loops), its bias gradient against the oracle's exact sum (the patterned
  inputs repeat, so the oracle runs over one period).

Inputs too large for the seeded CPU generator are deterministic patterns
computed on the device (and for the sampled rows, the same pattern on the
CPU): x[t, j] = ((t * H + j) mod 251 - 125) / 64, exactly representable.
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


def say(msg):
    print(f"[limits] {msg}", flush=True)


def pattern(rows, H, row0=0, device="cpu", dtype=torch.bfloat16, mod=251):
    """x[t, j] = ((t * H + j) mod `mod` - mod // 2) / 64, filled in row chunks
    (the int64 index temporaries of one chunk stay small)."""
    out = torch.empty((rows, H), dtype=dtype, device=device)
    j = torch.arange(H, device=device, dtype=torch.int64)[None, :]
    step = max(1, (1 << 24) // H)
    for a in range(0, rows, step):
        n = min(step, rows - a)
        t = torch.arange(row0 + a, row0 + a + n, device=device, dtype=torch.int64)[:, None]
        out[a:a + n] = (((t * H + j) % mod - (mod // 2)).to(torch.float32) / 64.0).to(dtype)
    return out


def test_mask_past_2_pow_34_elements():
    H = 64
    T = (1 << 28) + (1 << 14)  # 2^34 + 2^20 elements
    p, seed, off = 0.3, 987654321, 11
    bits = mb.mb_dropout_mask(T, H, p, seed, off)
    torch.cuda.synchronize()
    for r0 in (0, (1 << 28) - 3, T - 5):  # around the 2^34 boundary and the end
        n = 5
        ob = oracle.dropout_mask(n, H, p, seed, off, row0=r0)
        kb = bits[r0 * H // 8:(r0 + n) * H // 8].cpu().numpy()
        assert np.array_equal(kb, ob), f"mask bytes of rows {r0}..{r0 + n}"
    kept = torch.bitwise_and(bits[-(1 << 20):, None].to(torch.int32) >> torch.arange(8, device=DEV), 1).sum()
    frac = kept.item() / (8 << 20)
    assert abs(frac - 0.7) < 5 * np.sqrt(0.21 / (8 << 20))
    say(f"mask of {T * H} elements: sampled bytes equal; kept fraction of the last 2^23 elements {frac:.5f}")
    del bits


def test_dropout_add_past_2_pow_32_elements():
    H = 64
    T = (1 << 26) + (1 << 12)  # 2^32 + 2^18 elements, 8.6 GB per bf16 tensor
    p, seed, off = 0.1, 4242, 3
    x = pattern(T, H, device=DEV)
    r = pattern(T, H, device=DEV, mod=241)
    b = synthetic.draw(5, (H,), "normal", 0.02, "bf16")
    out = mb.mb_bias_dropout_add_train(x, b.to(DEV), r, p, seed, off)
    torch.cuda.synchronize()
    for r0 in (0, (1 << 26) - 2, T - 4):
        n = 4
        xs, rs = pattern(n, H, r0), pattern(n, H, r0, mod=241)
        assert torch.equal(xs, x[r0:r0 + n].cpu()) and torch.equal(rs, r[r0:r0 + n].cpu())
        o, o64, mag = oracle.bias_dropout_add("bf16", st(xs), st(b), st(rs), "bf16", True, p, seed, off, row0=r0)
        s = assert_close(st(out[r0:r0 + n]), o, o64, mag, "bf16", f"dropout-add rows {r0}")
        say(f"dropout-add {T}x{H} rows {r0}+{n}: {s}")
    del x, r, out


def test_gelu_widest_rows():
    strips = 65535
    H = strips * 64 * 8  # bf16: 8 elements per 16-byte vector
    T = 2
    y = synthetic.draw(11, (T, H), "normal", 2.0, "bf16").to(DEV)
    g = synthetic.draw(12, (T, H), "normal", 1.0, "bf16").to(DEV)
    b = synthetic.draw(13, (H,), "normal", 0.5, "bf16").to(DEV)
    out = mb.mb_bias_gelu_fwd(y, b)
    dg, db = mb.mb_bias_gelu_bwd(g, y, b)
    cols = torch.from_numpy(np.unique(np.concatenate([np.random.default_rng(3).choice(H, 4000, replace=False),
                                                      [0, 1, H - 8, H - 1]]))).to(DEV)
    ys, gs, bs = (st(t.index_select(-1, cols).cpu()) for t in (y, g, b))
    o, o64 = oracle.bias_gelu_fwd("bf16", ys, bs)
    s1 = assert_close(st(out.index_select(1, cols)), o, o64, None, "bf16", "gelu fwd widest rows")
    d, d64, mag, db64 = oracle.bias_gelu_bwd("bf16", gs, ys, bs)
    s2 = assert_close(st(dg.index_select(1, cols)), d, d64, mag, "bf16", "gelu bwd widest rows")
    assert_reduction_close(db.index_select(0, cols).cpu().numpy(), db64, "gelu dbias widest rows")
    say(f"gelu {T}x{H}: fwd {s1} bwd {s2}")
    with pytest.raises(mb.MBError):
        mb.mb_bias_gelu_fwd(torch.empty((1, H + 8), dtype=torch.bfloat16, device=DEV))  # one vector too many


def test_gelu_bwd_many_rows():
    """2^24 rows: a pattern of modulus m repeats every m rows (64 m = 0 mod
    m), so the two inputs together repeat every 251 * 239 = 59989 rows and the
    exact bias gradient is 279 times the oracle's over one period plus the
    oracle's over the first 40285 rows."""
    T, H = 1 << 24, 64
    P = 251 * 239
    y = pattern(T, H, device=DEV)
    g = pattern(T, H, device=DEV, mod=239)
    b = synthetic.draw(21, (H,), "normal", 0.02, "bf16").to(DEV)
    dg, db = mb.mb_bias_gelu_bwd(g, y, b)
    torch.cuda.synchronize()
    for r0 in (0, T // 2 + 1, T - 8):
        ys, gs = pattern(8, H, r0), pattern(8, H, r0, mod=239)
        d, d64, mag, _ = oracle.bias_gelu_bwd("bf16", st(gs), st(ys), st(b.cpu()))
        assert_close(st(dg[r0:r0 + 8]), d, d64, mag, "bf16", f"gelu bwd rows {r0}")
    full, rest = divmod(T, P)
    _, _, _, per = oracle.bias_gelu_bwd("bf16", st(pattern(P, H, mod=239)), st(pattern(P, H)), st(b.cpu()))
    _, _, _, part = oracle.bias_gelu_bwd("bf16", st(pattern(rest, H, mod=239)), st(pattern(rest, H)),
                                         st(b.cpu()))
    s = assert_reduction_close(db.cpu().numpy(), full * per + part, "gelu dbias over 2^24 rows")
    say(f"gelu bwd {T}x{H}: dbias {s}")
