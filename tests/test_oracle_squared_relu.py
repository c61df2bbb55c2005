"""Pins for the oracle's weighted squared ReLU (forward and backward).

- forward against torch's float64 CPU composition F.relu(x) ** 2 * w, and
  with w = None against F.relu(x) ** 2 (the unweighted op);
- backward against torch autograd in float64 (both dx and the per-token
  weights gradient) and against finite differences of the oracle's own
  forward (double storage);
- special values: negative inputs give 0 and a zero gradient, NaN passes
  through as torch's relu passes it, -inf gives 0;
- bf16 storage: every output is the once-rounded double.
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle


def rng(seed):
    return np.random.default_rng(seed)


@pytest.mark.parametrize("weighted", [True, False])
def test_forward_and_backward_match_torch_f64(weighted):
    r = rng(1)
    T, H = 7, 300
    x = r.normal(0, 2, (T, H))
    w = r.random(T) if weighted else None
    g = r.normal(0, 1, (T, H))
    out, out64 = oracle.weighted_squared_relu_fwd("f64", x, w)
    xt = torch.from_numpy(x).requires_grad_(True)
    wt = torch.from_numpy(w).requires_grad_(True) if weighted else None
    ref = F.relu(xt) ** 2 * (wt[:, None] if weighted else 1.0)
    np.testing.assert_allclose(out64, ref.detach().numpy(), rtol=1e-15, atol=0)
    (ref * torch.from_numpy(g)).sum().backward()
    dx, dx64, dw = oracle.weighted_squared_relu_bwd("f64", g, x, w)
    np.testing.assert_allclose(dx64, xt.grad.numpy(), rtol=1e-14, atol=0)
    if weighted:
        np.testing.assert_allclose(dw, wt.grad.numpy(), rtol=1e-12)
    else:
        assert dw is None


def test_finite_differences():
    r = rng(2)
    T, H = 3, 5
    x = r.normal(0, 1, (T, H))
    x[np.abs(x) < 0.05] = 0.3  # stay away from the kink at 0
    w = r.random(T) + 0.5
    g = r.normal(0, 1, (T, H))

    def L(x_, w_):
        _, o = oracle.weighted_squared_relu_fwd("f64", x_, w_)
        return float((g * o).sum())

    step = 1e-6
    fdx = np.zeros_like(x)
    for i in np.ndindex(*x.shape):
        a, b = x.copy(), x.copy()
        a[i] += step
        b[i] -= step
        fdx[i] = (L(a, w) - L(b, w)) / (2 * step)
    fdw = np.zeros_like(w)
    for t in range(T):
        a, b = w.copy(), w.copy()
        a[t] += step
        b[t] -= step
        fdw[t] = (L(x, a) - L(x, b)) / (2 * step)
    _, dx64, dw = oracle.weighted_squared_relu_bwd("f64", g, x, w)
    np.testing.assert_allclose(dx64, fdx, rtol=1e-6, atol=1e-8)
    np.testing.assert_allclose(dw, fdw, rtol=1e-6, atol=1e-8)


def test_special_values():
    x = np.array([[-3.0, -0.0, 0.0, 2.0, np.nan, -np.inf, np.inf, 1e-200]])
    w = np.array([0.5])
    _, o = oracle.weighted_squared_relu_fwd("f64", x, w)
    ref = F.relu(torch.from_numpy(x)) ** 2 * 0.5
    np.testing.assert_array_equal(np.isnan(o), np.isnan(ref.numpy()))
    fin = ~np.isnan(o)
    np.testing.assert_array_equal(o[fin], ref.numpy()[fin])
    assert o[0, 0] == 0.0 and o[0, 3] == 2.0 and np.isnan(o[0, 4]) and o[0, 5] == 0.0 and o[0, 6] == np.inf
    g = np.ones_like(x)
    _, d, _ = oracle.weighted_squared_relu_bwd("f64", g, x, w)
    assert d[0, 0] == 0.0 and d[0, 3] == 2.0 and np.isnan(d[0, 4]) and d[0, 5] == 0.0


def test_bf16_rounds_once():
    r = rng(3)
    T, H = 4, 256
    xf = r.normal(0, 3, (T, H)).astype(np.float32)
    x = torch.from_numpy(xf).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    w = r.random(T).astype(np.float32)
    out, out64 = oracle.weighted_squared_relu_fwd("bf16", x, w, "f32")
    once = np.array([oracle.round_bf16(v) for v in out64.reshape(-1)], np.uint16).reshape(T, H)
    assert np.array_equal(out, once)
    xv = torch.from_numpy(x.view(np.int16).copy()).view(torch.bfloat16).double()
    np.testing.assert_allclose(out64, (F.relu(xv) ** 2 * torch.from_numpy(w).double()[:, None]).numpy(), rtol=1e-15)


def test_rejects_dweights_without_weights():
    x = np.zeros((2, 4))
    assert oracle.weighted_squared_relu_bwd("f64", x, x, None)[2] is None
