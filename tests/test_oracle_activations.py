"""Pins for the oracle's activation functions.

- gelu_tanh / gelu_erf / silu against torch's float64 CPU implementations
  (a library routine; torch uses the exact sqrt(2/pi) and 1/sqrt(2), so the
  agreement is to the size of the printed constants' truncation);
- gelu_tanh and its derivative against an 80-digit decimal evaluation of the
  literal formulas, over the whole range including the negative tail where
  a double evaluation of the literal form cancels;
- analytic derivatives against central finite differences in double and
  against torch autograd in float64;
- the closed-form invariant that the tanh approximation stays within 1e-3 of
  the exact (erf) GeLU on [-6, 6].
"""
import json
import math
import os
from decimal import Decimal, getcontext

import numpy as np
import pytest
import scipy.special
import torch
import torch.nn.functional as F

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")
with open(os.path.join(GOLDEN, "page_constants.json")) as fh:
    CONST = {k: v["value"] for k, v in json.load(fh)["constants"].items()}

getcontext().prec = 80
DK = Decimal(CONST["sqrt_2_over_pi"])
DC = Decimal(CONST["cubic"])
DKG = Decimal(CONST["tanh_grad"])


def _dtanh(u: Decimal) -> Decimal:
    e = (2 * u).exp()
    return (e - 1) / (e + 1)


def _digits_for(z: float) -> int:
    # 1 + tanh(u) ~ 2 exp(2u) for u << 0: the literal form needs |2u| / ln(10)
    # extra digits to keep 60 significant ones
    u = 0.79788456 * z * (1 + 0.044715 * z * z)
    return 60 + int(abs(2 * u) / 2.302585) + 10


def dec_gelu_tanh(z: float) -> Decimal:
    getcontext().prec = _digits_for(z)
    z = Decimal(z)
    u = DK * z * (1 + DC * z * z)
    return Decimal("0.5") * z * (1 + _dtanh(u))


def dec_gelu_tanh_grad(z: float) -> Decimal:
    getcontext().prec = _digits_for(z)
    z = Decimal(z)
    u = DK * z * (1 + DC * z * z)
    t = _dtanh(u)
    return Decimal("0.5") * (1 + t) + Decimal("0.5") * z * (1 - t * t) * (DK + DKG * z * z)


def _rel(a, b):
    return abs(a - b) / max(abs(b), 1e-300)


ZS = np.concatenate([np.linspace(-12, 12, 2401), [-30.0, -20.0, 20.0, 30.0, -0.7525, 1e-8, -1e-8]])


def _cond_tol(z: float) -> Decimal:
    """Relative error bound of a double evaluation: exp(-2u) magnifies the
    rounding of u by |2u|, plus a few roundings elsewhere."""
    u = CONST["sqrt_2_over_pi"] * z * (1 + CONST["cubic"] * z * z)
    return Decimal(4e-16 * (2 * abs(u) + 20))


TINY = Decimal("1e-300")  # below this the double result underflows


def test_gelu_tanh_vs_80_digit_literal_formula():
    for z in ZS:
        want = dec_gelu_tanh(float(z))
        got = oracle.gelu_tanh(float(z))
        if abs(want) < TINY:
            assert abs(got) < 1e-300
            continue
        assert abs(Decimal(got) - want) <= _cond_tol(float(z)) * abs(want), (z, got, want)


def test_gelu_tanh_grad_vs_80_digit_literal_formula():
    for z in ZS:
        want = dec_gelu_tanh_grad(float(z))
        got = oracle.gelu_tanh_grad(float(z))
        if abs(want) < TINY:
            assert abs(got) < 1e-300
            continue
        # relative away from the derivative's root; near it, absolute against
        # the size of the summands (~0.3)
        assert abs(Decimal(got) - want) <= _cond_tol(float(z)) * abs(want) + Decimal("1e-16"), (z, got, want)


def test_gelu_tanh_vs_torch_float64():
    # torch evaluates the literal form in float64 with sqrt(2/pi) = 0.7978845608...;
    # the printed 0.79788456 differs by 1e-9 relative.
    z = np.linspace(-5, 8, 5001)
    ref = F.gelu(torch.from_numpy(z), approximate="tanh").numpy()
    for zi, r in zip(z, ref):
        got = oracle.gelu_tanh(float(zi))
        assert abs(got - r) <= 3e-8 * abs(r) + 1e-14, (zi, got, r)


def test_gelu_tanh_grad_vs_torch_autograd_float64():
    z = torch.linspace(-5, 8, 2001, dtype=torch.float64, requires_grad=True)
    F.gelu(z, approximate="tanh").sum().backward()
    for zi, r in zip(z.detach().numpy(), z.grad.numpy()):
        got = oracle.gelu_tanh_grad(float(zi))
        assert abs(got - r) <= 3e-8 * abs(r) + 3e-9, (zi, got, r)


def test_gelu_erf_vs_torch_and_scipy():
    z = np.linspace(-8, 8, 4001)
    ref_t = F.gelu(torch.from_numpy(z), approximate="none").numpy()
    ref_s = 0.5 * z * scipy.special.erfc(-z / math.sqrt(2.0))
    for zi, rt, rs in zip(z, ref_t, ref_s):
        got = oracle.gelu_erf(float(zi))
        # 0.70710678 vs 1/sqrt(2): 1.7e-9 relative in the argument, magnified
        # by about z^2 in the erfc tail
        tol = 2e-9 * (zi * zi + 2)
        assert abs(got - rs) <= tol * abs(rs) + 1e-15, (zi, got, rs)
        assert abs(got - rt) <= tol * abs(rt) + 1e-15, (zi, got, rt)


def test_gelu_erf_grad_vs_torch_autograd():
    z = torch.linspace(-8, 8, 2001, dtype=torch.float64, requires_grad=True)
    F.gelu(z, approximate="none").sum().backward()
    for zi, r in zip(z.detach().numpy(), z.grad.numpy()):
        got = oracle.gelu_erf_grad(float(zi))
        # 0.3989423 is 1/sqrt(2 pi) to 7 digits: 5e-8 relative in the second
        # term (at most ~0.25 in size); 0.70710678 as above in the first
        assert abs(got - r) <= 3e-8 + 2e-9 * (float(zi) ** 2 + 2) * abs(r), (zi, got, r)


def test_silu_vs_torch_float64():
    a = np.linspace(-40, 40, 8001)
    ref = F.silu(torch.from_numpy(a)).numpy()
    for ai, r in zip(a, ref):
        got = oracle.silu(float(ai))
        assert abs(got - r) <= 1e-15 * abs(r) + 1e-300, (ai, got, r)


def test_silu_grad_vs_torch_autograd_float64():
    a = torch.linspace(-30, 15, 4501, dtype=torch.float64, requires_grad=True)
    F.silu(a).sum().backward()
    for ai, r in zip(a.detach().numpy(), a.grad.numpy()):
        got = oracle.silu_grad(float(ai))
        assert abs(got - r) <= 1e-12 * abs(r) + 1e-15, (ai, got, r)


def _fd(f, z):
    h = 1e-5 * max(1.0, abs(z))
    return (f(z + h) - f(z - h)) / (2 * h)


@pytest.mark.parametrize("fwd,grad", [
    (oracle.gelu_tanh, oracle.gelu_tanh_grad),
    (oracle.gelu_erf, oracle.gelu_erf_grad),
    (oracle.silu, oracle.silu_grad),
])
def test_derivative_vs_central_differences(fwd, grad):
    for z in np.linspace(-9, 9, 1801):
        z = float(z)
        fd = _fd(fwd, z)
        an = grad(z)
        # central differences: truncation ~h^2 f'''/6, rounding ~1e-16/h
        # The erf GeLU's printed constants 0.70710678 and 0.3989423 agree with
        # each other only to ~5e-8, so its derivative gets that much slack.
        slack = 3e-8 if fwd is oracle.gelu_erf else 0.0
        assert abs(an - fd) <= 1e-7 * max(abs(fd), 1e-3) + slack, (fwd.__name__, z, an, fd)


def test_tanh_gelu_within_1e3_of_erf_gelu():
    z = np.linspace(-6, 6, 120001)
    d = np.array([oracle.gelu_tanh(float(v)) - oracle.gelu_erf(float(v)) for v in z])
    worst = float(np.max(np.abs(d)))
    assert worst <= 1e-3
    # and the two are genuinely different functions (the approximation error is ~5e-4)
    assert worst >= 1e-4
    zw = abs(float(z[int(np.argmax(np.abs(d)))]))
    assert 2.0 < zw < 3.5


def test_tanh_grad_constant_is_product_of_printed_constants():
    # the page states 0.1070322243 = sqrt(2/pi) * 3 * 0.044715
    assert abs(CONST["tanh_grad"] - CONST["sqrt_2_over_pi"] * 3 * CONST["cubic"]) < 1e-10
    assert abs(CONST["sqrt_2_over_pi"] - math.sqrt(2 / math.pi)) < 1e-8
    assert abs(CONST["inv_sqrt_2"] - 1 / math.sqrt(2)) < 1e-8
    assert abs(CONST["inv_sqrt_2pi"] - 1 / math.sqrt(2 * math.pi)) < 1e-7


def test_special_values():
    assert oracle.gelu_tanh(0.0) == 0.0
    assert oracle.gelu_tanh_grad(0.0) == 0.5
    assert oracle.silu(0.0) == 0.0
    assert oracle.silu_grad(0.0) == 0.5
    assert math.isnan(oracle.gelu_tanh(math.nan))
    assert math.isnan(oracle.gelu_tanh_grad(math.nan))
    assert oracle.gelu_tanh(1e6) == 1e6
    assert oracle.gelu_tanh_grad(1e6) == 1.0
    assert oracle.gelu_tanh(-1e6) == 0.0 and oracle.gelu_tanh_grad(-1e6) == 0.0
