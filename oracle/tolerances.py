"""Parity comparators between kernel outputs and the oracle (test
infrastructure, like the rest of this package).

Floating point (per element, kernel value k, oracle value o rounded once to
the output dtype, unrounded oracle value o64):
  fp32 outputs:       |k - o| <= 1e-6 |o| + 1e-6
  bf16/fp16 outputs:  |k - o| <= 1 ulp_dt(o)
  either, at cancellations only: |k - o64| <= 8 * 2^-24 * mag, where mag is
      the size of the largest term the fp32 evaluation combines (reported
      separately as "floor" passes; it only matters near roots of the
      derivatives and where r' + z*s cancels, and for fp32 outputs only when
      an upstream factor (the gradient, the up half) scales such a root
      value far above the 1e-6 absolute term)
  fp32 reductions (dbias, dweights): |k - o| <= 1e-3 |o| + 1e-3 rms(o)
Integers / bits: exact. Equal bit patterns, both NaN, and +0 vs -0 pass.
The statistics count the passes that needed the cancellation floor
("floor_only") and, for fp32, the 1e-6 absolute term ("abs_only": a value
below about 1e-4 in magnitude off by more than 1e-6 relative); callers on
natural data bound both (assert_close's max_floor_frac and max_abs_only).
"""
from __future__ import annotations

import numpy as np
import torch

FLOOR_FACTOR = 8 * 2.0**-24


def to_storage(t: torch.Tensor) -> np.ndarray:
    """Raw storage of a CPU/GPU tensor in the oracle's convention."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype in (torch.bfloat16, torch.float16):
        return t.view(torch.int16).numpy().view(np.uint16)
    raise TypeError(t.dtype)


def from_storage(a: np.ndarray, dtype: torch.dtype) -> torch.Tensor:
    if dtype == torch.float32:
        return torch.from_numpy(np.ascontiguousarray(a, np.float32))
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(dtype)


def values(a: np.ndarray, dt: str) -> np.ndarray:
    if dt == "f32":
        return a.astype(np.float64)
    t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16).copy()).view(
        torch.bfloat16 if dt == "bf16" else torch.float16)
    return t.to(torch.float64).numpy()


def ulp(o: np.ndarray, dt: str) -> np.ndarray:
    """Spacing of the dt grid at |o| (the subnormal spacing below the normal range)."""
    prec, emin = (8, -126) if dt == "bf16" else (11, -14)
    a = np.abs(o)
    with np.errstate(divide="ignore"):
        e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    e = np.maximum(np.where(a > 0, e, emin), emin)
    return np.ldexp(1.0, (e - (prec - 1)).astype(np.int64))


def compare(kernel: np.ndarray, oracle_out: np.ndarray, o64: np.ndarray, mag, dt: str, cond=None):
    """Returns (pass mask, stats dict).

    cond (per element, or None): the size |E| of the exponent the function
    takes (2|u| for the tanh GeLU, z^2/2 for the exact one, |a| for SiLU), the
    relative condition of exp(E) to the rounding of its argument. With it the
    fp32 rule is the pure relative 1e-6 bound, and the floor is
    8 * 2^-24 * (1 + cond) * mag (mag = |o64| when the op has none): an fp32
    evaluation rounds E, so its result carries about |E| 2^-24 relative error
    in the tail, where 1e-6 relative is out of reach for any fp32 kernel. The
    1e-6 absolute term is not used then."""
    k = values(kernel, dt)
    o = values(oracle_out, dt)
    same_bits = kernel.view(np.uint32 if dt == "f32" else np.uint16) == oracle_out.view(
        np.uint32 if dt == "f32" else np.uint16)
    both_nan = np.isnan(k) & np.isnan(o)
    with np.errstate(invalid="ignore"):
        d = np.abs(k - o)
        d = np.where(np.isinf(k) & np.isinf(o) & (np.sign(k) == np.sign(o)), 0.0, d)
        rel_ok = d <= 1e-6 * np.abs(o) if dt == "f32" else d <= ulp(o, dt)
        if cond is None:
            ok = d <= 1e-6 * np.abs(o) + 1e-6 if dt == "f32" else rel_ok
            floor = FLOOR_FACTOR * (mag if mag is not None else 0.0)
        else:
            ok = rel_ok
            floor = FLOOR_FACTOR * (1.0 + np.abs(cond)) * (mag if mag is not None else np.abs(o64))
        floor_ok = ~ok & (np.abs(k - o64) <= floor)
    passed = same_bits | both_nan | ok | floor_ok
    with np.errstate(invalid="ignore", divide="ignore"):
        rel = np.where(np.abs(o) > 0, d / np.abs(o), 0.0)
        ulps = d / ulp(o, dt) if dt != "f32" else rel
    fin = np.isfinite(ulps)
    stats = {
        "n": int(k.size),
        "fail": int((~passed).sum()),
        "bit_equal": int(same_bits.sum()),
        "floor_only": int((floor_ok & ~ok & ~same_bits).sum()),
        "abs_only": int((ok & ~rel_ok & ~same_bits & ~both_nan).sum()),
        "max_ulp_or_rel": float(np.max(ulps[fin])) if fin.any() else 0.0,
        "max_abs": float(np.nanmax(d)) if d.size else 0.0,
        "ref_max": float(np.nanmax(np.abs(o))) if o.size else 0.0,
    }
    return passed, stats


def assert_close(kernel, oracle_out, o64, mag, dt, what="", max_floor_frac=None, max_abs_only=None, cond=None):
    """Per-element parity; max_floor_frac bounds the fraction of floor-only
    passes, max_abs_only the count of passes on the fp32 absolute term alone;
    cond as for compare."""
    passed, stats = compare(kernel, oracle_out, o64, mag, dt, cond)
    if max_floor_frac is not None and stats["floor_only"] > max(1, max_floor_frac * stats["n"]):
        raise AssertionError(f"{what}: {stats['floor_only']}/{stats['n']} passes needed the cancellation floor "
                             f"(more than {max_floor_frac:g} of the elements); stats {stats}")
    if max_abs_only is not None and stats["abs_only"] > max_abs_only:
        raise AssertionError(f"{what}: {stats['abs_only']} fp32 passes needed the absolute term; stats {stats}")
    if stats["fail"]:
        idx = np.flatnonzero(~passed.reshape(-1))[:8]
        kv, ov = values(kernel, dt).reshape(-1), values(oracle_out, dt).reshape(-1)
        ex = [(int(i), float(kv[i]), float(ov[i]), float(o64.reshape(-1)[i])) for i in idx]
        raise AssertionError(f"{what}: {stats['fail']}/{stats['n']} elements out of tolerance; "
                             f"first (index, kernel, oracle, oracle64): {ex}; stats {stats}")
    return stats


def assert_reduction_close(kernel: np.ndarray, oracle64: np.ndarray, what=""):
    k = kernel.astype(np.float64)
    o = oracle64
    rms = float(np.sqrt(np.mean(o * o))) if o.size else 0.0
    bad = np.abs(k - o) > 1e-3 * np.abs(o) + 1e-3 * rms
    if bad.any():
        i = np.flatnonzero(bad)[:8]
        raise AssertionError(f"{what}: {int(bad.sum())}/{o.size} out of 1e-3 tolerance; first {list(zip(i, k[i], o[i]))}")
    worst = float(np.max(np.abs(k - o) / (np.abs(o) + rms + 1e-300))) if o.size else 0.0
    return {"n": int(o.size), "max_rel_to_rms": worst}


def assert_close_bounded(kernel, oracle_out, o64, bound, dt, what=""):
    """For ops whose fp32 evaluation error has a derived bound per element
    (row reductions such as LayerNorm): passes when the bits are equal, both
    are NaN, |k - o| <= 1 ulp of the once-rounded oracle value (bf16/fp16), or
    |k - o64| <= bound + the output rounding (half an fp32 ulp, one bf16/fp16
    ulp)."""
    k = values(kernel, dt)
    o = values(oracle_out, dt)
    same_bits = kernel.view(np.uint32 if dt == "f32" else np.uint16) == oracle_out.view(
        np.uint32 if dt == "f32" else np.uint16)
    both_nan = np.isnan(k) & np.isnan(o)
    with np.errstate(invalid="ignore"):
        if dt == "f32":
            ok = np.abs(k - o64) <= bound + 2.0**-24 * np.abs(o64)
        else:
            ok = (np.abs(k - o) <= ulp(o, dt)) | (np.abs(k - o64) <= bound + ulp(o64, dt))
    passed = same_bits | both_nan | ok
    err = np.abs(k - o64)
    with np.errstate(invalid="ignore", divide="ignore"):
        ratio = np.where(bound > 0, err / bound, 0.0)
    stats = {"n": int(k.size), "fail": int((~passed).sum()), "bit_equal": int(same_bits.sum()),
             "max_err_over_bound": float(np.nanmax(ratio)) if ratio.size else 0.0,
             "max_abs": float(np.nanmax(err)) if err.size else 0.0}
    if stats["fail"]:
        idx = np.flatnonzero(~passed.reshape(-1))[:8]
        ex = [(int(i), float(k.reshape(-1)[i]), float(o64.reshape(-1)[i]), float(np.reshape(bound, -1)[i]))
              for i in idx]
        raise AssertionError(f"{what}: {stats['fail']}/{stats['n']} out of bound; first (index, kernel, oracle64, "
                             f"bound): {ex}; stats {stats}")
    return stats
