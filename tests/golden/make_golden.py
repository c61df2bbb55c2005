"""Writes tests/golden/oracle_regression.json: small seeded cases evaluated by
the oracle alone (nothing else is imported), stored as raw bit patterns, so
that any later change to the oracle's arithmetic shows up as a diff.

Run from the repository root:  python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)
import oracle  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_regression.json")


def bf16_from_f32(a):
    """Round float32 values to bf16 bit patterns with the oracle's rounding."""
    return np.array([oracle.round_bf16(float(v)) for v in a.reshape(-1)], np.uint16).reshape(a.shape)


def hexs(a):
    a = np.ascontiguousarray(a)
    if a.dtype == np.float64:
        return [float(v).hex() for v in a.reshape(-1)]
    return [int(v) for v in a.view(np.uint16 if a.dtype == np.uint16 else np.uint32).reshape(-1)]


def main():
    r = np.random.default_rng(20240601)
    cases = []
    T, H = 4, 8
    y = bf16_from_f32(r.standard_normal((T, H)).astype(np.float32) * 2)
    g = bf16_from_f32(r.standard_normal((T, H)).astype(np.float32))
    b = bf16_from_f32((r.standard_normal(H) * 0.1).astype(np.float32))
    out, _ = oracle.bias_gelu_fwd("bf16", y, b)
    dg, _, _, db = oracle.bias_gelu_bwd("bf16", g, y, b)
    cases.append({"op": "gelu", "dt": "bf16", "T": T, "H": H, "y": hexs(y), "g": hexs(g), "bias": hexs(b),
                  "out": hexs(out), "dgrad": hexs(dg), "dbias": hexs(db)})
    x = bf16_from_f32(r.standard_normal((T, H)).astype(np.float32))
    res = r.standard_normal((T, H)).astype(np.float32)
    tr, _, _ = oracle.bias_dropout_add("bf16", x, b, res, "f32", True, 0.1, 1234, 0)
    inf, _, _ = oracle.bias_dropout_add("bf16", x, b, res, "f32", False)
    mask = oracle.dropout_mask(T, H, 0.5, 1234, 3)
    cases.append({"op": "bda", "dt": "bf16", "T": T, "H": H, "x": hexs(x), "bias": hexs(b),
                  "residual_f32": hexs(res), "p": 0.1, "seed": 1234, "offset": 0,
                  "train": hexs(tr), "infer": hexs(inf), "mask_p05_off3": [int(v) for v in mask]})
    xin = bf16_from_f32(r.standard_normal((T, 2 * H)).astype(np.float32) * 2)
    b2 = bf16_from_f32((r.standard_normal(2 * H) * 0.1).astype(np.float32))
    w = bf16_from_f32(r.random(T).astype(np.float32))
    for act in ("swiglu", "geglu"):
        wt = w if act == "swiglu" else None
        o, _ = oracle.bias_glu_fwd(act, "bf16", xin, b2, wt)
        d, _, _, dbb, dw = oracle.bias_glu_bwd(act, "bf16", g, xin, b2, wt)
        c = {"op": act, "dt": "bf16", "T": T, "H": H, "in": hexs(xin), "bias": hexs(b2), "g": hexs(g),
             "out": hexs(o), "din": hexs(d), "dbias": hexs(dbb)}
        if wt is not None:
            c["weights"] = hexs(wt)
            c["dweights"] = hexs(dw)
        cases.append(c)
    with open(OUT, "w") as fh:
        json.dump({"generator": "tests/golden/make_golden.py (oracle only)", "cases": cases}, fh, indent=0)
    print("wrote", OUT)


if __name__ == "__main__":
    main()
