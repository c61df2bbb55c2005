"""Pins for the oracle's residual add + LayerNorm (forward and backward).

- forward against torch's CPU LayerNorm in float64 (F.layer_norm, the
  biased variance, eps inside the square root), with and without the
  zero-centred gamma (weight + 1), including rows whose variance is close to
  eps so that a misplaced or missing eps shows;
- the residual add against torch's own dtype arithmetic (bf16 + cast residual);
- bf16 outputs equal torch's float64 LayerNorm rounded once;
- closed form at H = 2, and H = 1 (y = beta, dx = dh_in);
- invariants with eps = 0: shift and scale invariance, mean(xhat) = 0,
  mean(xhat^2) = 1;
- backward against torch autograd in float64 and against a finite-difference
  gradient of the oracle's own forward (double storage) over every input,
  gamma and beta element of small tensors, with an upstream gradient on h.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rng(seed):
    return np.random.default_rng(seed)


def bf16_bits(a):
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def bf16_tensor(bits):
    return torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16)


def torch_ln(h64, g64, b64, eps, zero_centered):
    w = torch.from_numpy(g64) + (1.0 if zero_centered else 0.0)
    b = torch.from_numpy(b64) if b64 is not None else None
    return F.layer_norm(torch.from_numpy(h64), (h64.shape[1],), w, b, eps).numpy()


@pytest.mark.parametrize("zero_centered", [False, True])
@pytest.mark.parametrize("T,H,scale,shift", [(3, 64, 1.0, 0.0), (5, 1000, 3.0, 7.0), (4, 256, 2e-3, 0.5),
                                            (2, 4096, 1.0, -2.0)])
def test_forward_matches_torch_f64(T, H, scale, shift, zero_centered):
    r = rng(T * H)
    x = r.normal(0, scale, (T, H)) + shift
    res = r.normal(0, scale, (T, H))
    g = r.normal(0, 0.5, H) + (0.0 if zero_centered else 1.0)
    b = r.normal(0, 0.3, H)
    h, y, y64, mag, mean, rstd = oracle.add_layer_norm_fwd("f64", x, res, "f64", g, b, 1e-5, zero_centered)
    hh = x + res
    assert np.array_equal(h, hh)
    ref = torch_ln(hh, g, b, np.float32(1e-5).item(), zero_centered)
    np.testing.assert_allclose(y64, ref, rtol=1e-10, atol=1e-10)
    var, mu = torch.var_mean(torch.from_numpy(hh), dim=1, unbiased=False)
    np.testing.assert_allclose(mean, mu.numpy(), rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(rstd, 1.0 / np.sqrt(var.numpy() + np.float32(1e-5)), rtol=1e-12)
    assert np.all(np.abs(y64) <= mag * (1 + 1e-12))


def test_eps_matters_at_small_variance():
    r = rng(1)
    x = r.normal(0, 1e-3, (2, 128))
    g = np.ones(128)
    _, _, y_a, _, _, _ = oracle.add_layer_norm_fwd("f64", x, np.zeros_like(x), "f64", g, None, 1e-5)
    _, _, y_b, _, _, _ = oracle.add_layer_norm_fwd("f64", x, np.zeros_like(x), "f64", g, None, 0.0)
    # var ~ 1e-6: eps = 1e-5 shrinks the output by sqrt(var / (var + eps)) ~ 0.3
    ratio = np.abs(y_a).sum() / np.abs(y_b).sum()
    assert 0.2 < ratio < 0.5
    ref = torch_ln(x, g, None, np.float32(1e-5).item(), False)
    np.testing.assert_allclose(y_a, ref, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("res_dt", ["bf16", "f32"])
def test_bf16_residual_add_and_single_rounding(res_dt):
    T, H = 6, 512
    r = rng(7)
    xf = r.normal(0, 2, (T, H)).astype(np.float32)
    rf = (r.normal(0, 2, (T, H)) * np.where(r.random((T, H)) < 0.1, 1e3, 1.0)).astype(np.float32)
    gf = r.normal(1, 0.2, H).astype(np.float32)
    bf = r.normal(0, 0.2, H).astype(np.float32)
    x, g, b = bf16_bits(xf), bf16_bits(gf), bf16_bits(bf)
    res = bf16_bits(rf) if res_dt == "bf16" else rf
    h, y, y64, _, _, _ = oracle.add_layer_norm_fwd("bf16", x, res, res_dt, g, b, 1e-5)
    res_t = bf16_tensor(res) if res_dt == "bf16" else torch.from_numpy(rf)
    h_ref = bf16_tensor(x) + res_t.to(torch.bfloat16)  # torch's bf16 add: exact sum, rounded once
    assert np.array_equal(h, h_ref.view(torch.int16).numpy().view(np.uint16))
    y_ref = F.layer_norm(h_ref.double(), (H,), bf16_tensor(g).double(), bf16_tensor(b).double(),
                         np.float32(1e-5).item())
    np.testing.assert_allclose(y64, y_ref.numpy(), rtol=1e-10, atol=1e-10)
    assert np.array_equal(y, y_ref.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16))


def test_closed_form_h2_and_h1():
    a, c, eps = 3.0, -1.0, 1e-5
    x = np.array([[a, c]])
    g = np.array([1.5, -0.5])
    b = np.array([0.25, 2.0])
    _, _, y, _, mean, rstd = oracle.add_layer_norm_fwd("f64", x, np.zeros_like(x), "f64", g, b, eps)
    d = (a - c) / 2
    e32 = float(np.float32(eps))
    s = d / np.sqrt(d * d + e32)
    np.testing.assert_allclose(y[0], [g[0] * s + b[0], -g[1] * s + b[1]], rtol=1e-14)
    assert mean[0] == 1.0 and abs(rstd[0] - 1 / np.sqrt(d * d + e32)) < 1e-15
    # H = 1: the row is its own mean, y = beta; the gradient through the
    # normalisation vanishes and only the upstream term remains
    x1 = np.array([[5.0], [-2.0]])
    _, _, y1, _, _, _ = oracle.add_layer_norm_fwd("f64", x1, np.zeros_like(x1), "f64", np.array([3.0]),
                                                  np.array([0.5]), eps)
    assert np.all(y1 == 0.5)
    dx, _, _, _, dgam, dbet = oracle.add_layer_norm_bwd("f64", np.array([[1.0], [2.0]]), x1, np.array([3.0]), eps,
                                                        dh_in=np.array([[0.25], [-4.0]]))
    assert np.array_equal(dx, np.array([[0.25], [-4.0]]))
    assert dgam[0] == 0.0 and dbet[0] == 3.0


def test_invariants_eps0():
    r = rng(3)
    T, H = 4, 300
    x = r.normal(0, 1, (T, H))
    g = np.ones(H)
    _, _, y, _, _, _ = oracle.add_layer_norm_fwd("f64", x, np.zeros_like(x), "f64", g, None, 0.0)
    np.testing.assert_allclose(y.mean(1), 0.0, atol=1e-13)
    np.testing.assert_allclose((y * y).mean(1), 1.0, rtol=1e-12)
    _, _, y2, _, _, _ = oracle.add_layer_norm_fwd("f64", 7.5 * x - 3.0, np.zeros_like(x), "f64", g, None, 0.0)
    np.testing.assert_allclose(y2, y, rtol=1e-11, atol=1e-11)


def test_zero_centered_equals_weight_plus_one():
    r = rng(4)
    x = r.normal(0, 1, (3, 128))
    g = r.normal(0, 0.1, 128)
    b = r.normal(0, 0.1, 128)
    _, _, y1, _, _, _ = oracle.add_layer_norm_fwd("f64", x, np.zeros_like(x), "f64", g, b, 1e-5, True)
    _, _, y2, _, _, _ = oracle.add_layer_norm_fwd("f64", x, np.zeros_like(x), "f64", g + 1.0, b, 1e-5, False)
    np.testing.assert_allclose(y1, y2, rtol=1e-14, atol=1e-15)


@pytest.mark.parametrize("zero_centered", [False, True])
def test_backward_matches_torch_autograd(zero_centered):
    r = rng(5)
    T, H = 5, 384
    x = r.normal(0.3, 1.5, (T, H))
    res = r.normal(0, 1, (T, H))
    g = r.normal(0, 0.4, H) + (0.0 if zero_centered else 1.0)
    b = r.normal(0, 0.2, H)
    dy = r.normal(0, 1, (T, H))
    up = r.normal(0, 0.5, (T, H))
    h = x + res
    eps = float(np.float32(1e-5))
    ht = torch.from_numpy(h).requires_grad_(True)
    gt = torch.from_numpy(g).requires_grad_(True)
    bt = torch.from_numpy(b).requires_grad_(True)
    yt = F.layer_norm(ht, (H,), gt + (1.0 if zero_centered else 0.0), bt, eps)
    (yt * torch.from_numpy(dy)).sum().backward()
    dx, dx64, mag, dres, dgam, dbet = oracle.add_layer_norm_bwd("f64", dy, h, g, 1e-5, zero_centered, dh_in=up)
    np.testing.assert_allclose(dx64, ht.grad.numpy() + up, rtol=1e-10, atol=1e-11)
    np.testing.assert_allclose(dgam, gt.grad.numpy(), rtol=1e-10, atol=1e-10)
    np.testing.assert_allclose(dbet, bt.grad.numpy(), rtol=1e-12, atol=1e-12)
    assert np.array_equal(dres, dx)
    assert np.all(np.abs(dx64) <= mag * (1 + 1e-12))


def test_backward_finite_differences():
    """Gradient of L = sum(dy * y) + sum(up * h) with respect to x, gamma and
    beta by central differences of the oracle's forward (double storage)."""
    r = rng(6)
    T, H = 2, 6
    x = r.normal(0, 1, (T, H))
    res = r.normal(0, 1, (T, H))
    g = r.normal(1, 0.3, H)
    b = r.normal(0, 0.3, H)
    dy = r.normal(0, 1, (T, H))
    up = r.normal(0, 1, (T, H))

    def L(x_, g_, b_):
        h, _, y64, _, _, _ = oracle.add_layer_norm_fwd("f64", x_, res, "f64", g_, b_, 1e-5)
        return float((dy * y64).sum() + (up * h).sum())

    step = 1e-6
    fd_x = np.zeros_like(x)
    for i in np.ndindex(*x.shape):
        xp, xm = x.copy(), x.copy()
        xp[i] += step
        xm[i] -= step
        fd_x[i] = (L(xp, g, b) - L(xm, g, b)) / (2 * step)
    fd_g = np.zeros_like(g)
    fd_b = np.zeros_like(b)
    for j in range(H):
        gp, gm, bp, bm = g.copy(), g.copy(), b.copy(), b.copy()
        gp[j] += step
        gm[j] -= step
        bp[j] += step
        bm[j] -= step
        fd_g[j] = (L(x, gp, b) - L(x, gm, b)) / (2 * step)
        fd_b[j] = (L(x, g, bp) - L(x, g, bm)) / (2 * step)
    dx, dx64, _, dres, dgam, dbet = oracle.add_layer_norm_bwd("f64", dy, x + res, g, 1e-5, dh_in=up)
    np.testing.assert_allclose(dx64, fd_x, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dgam, fd_g, rtol=1e-6, atol=1e-7)
    np.testing.assert_allclose(dbet, fd_b, rtol=1e-6, atol=1e-7)


def test_backward_dtypes_round_once():
    r = rng(8)
    T, H = 3, 256
    hf = r.normal(0, 1, (T, H)).astype(np.float32)
    h = bf16_bits(hf)
    g = bf16_bits(r.normal(1, 0.1, H).astype(np.float32))
    dy = bf16_bits(r.normal(0, 1, (T, H)).astype(np.float32))
    up = r.normal(0, 1, (T, H)).astype(np.float32)
    dx, dx64, _, dres, _, _ = oracle.add_layer_norm_bwd("bf16", dy, h, g, 1e-5, dh_in=up, res_dt="f32")
    assert np.array_equal(dres, dx64.astype(np.float32))
    # the bf16 gradient is the once-rounded double (the rounding routine is
    # pinned on its own in test_oracle_formats.py)
    once = np.array([oracle.round_bf16(v) for v in dx64.reshape(-1)], np.uint16).reshape(T, H)
    assert np.array_equal(dx, once)


def test_rejects_bad_arguments():
    x = np.zeros((2, 4))
    with pytest.raises(ValueError):
        oracle.add_layer_norm_fwd("f64", x, x, "f64", np.ones(4), None, -1.0)
    with pytest.raises(ValueError):
        oracle.add_layer_norm_fwd("f64", x, x, "f64", np.ones(4), None, float("nan"))
