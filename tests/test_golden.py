"""Stored fixtures: the page's printed constants and the oracle regression cases.

page_constants.json holds the constants exactly as the fusions article prints
them (section 4.2); oracle_regression.json was written by
tests/golden/make_golden.py, which calls only the oracle. Any change to the
oracle's arithmetic changes these bits and must be justified by the passage
it follows.
"""
import json
import os

import numpy as np

import oracle

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _u16(v, shape):
    return np.array(v, np.uint16).reshape(shape)


def _f64(v):
    return np.array([float.fromhex(s) for s in v])


def test_page_constants_fixture():
    with open(os.path.join(GOLDEN, "page_constants.json")) as fh:
        c = {k: v["value"] for k, v in json.load(fh)["constants"].items()}
    assert c == {"sqrt_2_over_pi": 0.79788456, "cubic": 0.044715, "tanh_grad": 0.1070322243,
                 "inv_sqrt_2": 0.70710678, "inv_sqrt_2pi": 0.3989423}
    # the oracle's derivative at 0 is 0.5 and its second-order behaviour uses
    # the printed sqrt(2/pi): gelu'(z) ~ 0.5 + sqrt(2/pi) z for small z
    z = 1e-4
    slope = (oracle.gelu_tanh_grad(z) - oracle.gelu_tanh_grad(-z)) / (2 * z)
    assert abs(slope - c["sqrt_2_over_pi"]) < 1e-6


def test_oracle_regression_cases():
    with open(os.path.join(GOLDEN, "oracle_regression.json")) as fh:
        cases = json.load(fh)["cases"]
    for c in cases:
        T, H = c["T"], c["H"]
        if c["op"] == "gelu":
            y, g, b = _u16(c["y"], (T, H)), _u16(c["g"], (T, H)), _u16(c["bias"], (H,))
            out, _ = oracle.bias_gelu_fwd("bf16", y, b)
            dg, _, _, db = oracle.bias_gelu_bwd("bf16", g, y, b)
            assert out.reshape(-1).tolist() == c["out"]
            assert dg.reshape(-1).tolist() == c["dgrad"]
            assert np.array_equal(db, _f64(c["dbias"]))
        elif c["op"] == "bda":
            x, b = _u16(c["x"], (T, H)), _u16(c["bias"], (H,))
            res = np.array(c["residual_f32"], np.uint32).view(np.float32).reshape(T, H)
            tr, _, _ = oracle.bias_dropout_add("bf16", x, b, res, "f32", True, c["p"], c["seed"], c["offset"])
            inf, _, _ = oracle.bias_dropout_add("bf16", x, b, res, "f32", False)
            assert tr.reshape(-1).tolist() == c["train"]
            assert inf.reshape(-1).tolist() == c["infer"]
            assert oracle.dropout_mask(T, H, 0.5, 1234, 3).tolist() == c["mask_p05_off3"]
        else:
            xin, b2, g = _u16(c["in"], (T, 2 * H)), _u16(c["bias"], (2 * H,)), _u16(c["g"], (T, H))
            w = _u16(c["weights"], (T,)) if "weights" in c else None
            o, _ = oracle.bias_glu_fwd(c["op"], "bf16", xin, b2, w)
            d, _, _, dbb, dw = oracle.bias_glu_bwd(c["op"], "bf16", g, xin, b2, w)
            assert o.reshape(-1).tolist() == c["out"]
            assert d.reshape(-1).tolist() == c["din"]
            assert np.array_equal(dbb, _f64(c["dbias"]))
            if w is not None:
                assert np.array_equal(dw, _f64(c["dweights"]))
