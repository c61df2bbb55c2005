"""Pins for the oracle's number-format code: decoding and round-once-to-nearest-even.

Pinned against (a) torch's and numpy's CPU conversions, exhaustively over
all 65536 16-bit patterns for decoding, and (b) exact rational brute force
(the two neighbouring representable values, nearest wins, ties to even) for
rounding from double, where torch itself would round twice.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def _same(a: float, b: float) -> bool:
    return (math.isnan(a) and math.isnan(b)) or (a == b and math.copysign(1, a) == math.copysign(1, b))


def test_decode_bf16_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ref = torch.from_numpy(bits.view(np.int16).copy()).view(torch.bfloat16).to(torch.float64).numpy()
    got = oracle.decode("bf16", bits)
    for a, b in zip(got, ref):
        assert _same(float(a), float(b))


def test_decode_f16_exhaustive():
    bits = np.arange(65536, dtype=np.uint16)
    ref = bits.view(np.float16).astype(np.float64)
    got = oracle.decode("f16", bits)
    for a, b in zip(got, ref):
        assert _same(float(a), float(b))


def _rand_floats(n, seed):
    rng = np.random.default_rng(seed)
    raw = rng.integers(0, 2**32, size=n, dtype=np.uint64).astype(np.uint32)
    f = raw.view(np.float32)
    special = np.array([0.0, -0.0, np.inf, -np.inf, np.nan, 1e-45, -1e-45, 1.17549435e-38,
                        3.3895314e38, 3.4028235e38, 65504.0, 65519.99, 65520.0, 6.0e-8, 2.98e-8,
                        1.0, 1.00390625, 1.005859375, 1.001953125], np.float32)
    return np.concatenate([f, special])


def test_round_bf16_from_float_matches_torch():
    f = _rand_floats(20000, 1)
    ref = torch.from_numpy(f).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    for v, r in zip(f, ref):
        got = oracle.round_bf16(float(v))
        if math.isnan(v):
            assert (got & 0x7F80) == 0x7F80 and (got & 0x7F) != 0
        else:
            assert got == int(r), (float(v), hex(got), hex(int(r)))


def test_round_f16_from_float_matches_torch_and_numpy():
    f = _rand_floats(20000, 2)
    ref_t = torch.from_numpy(f).to(torch.float16).view(torch.int16).numpy().view(np.uint16)
    ref_n = f.astype(np.float16).view(np.uint16)
    for v, rt, rn in zip(f, ref_t, ref_n):
        got = oracle.round_f16(float(v))
        if math.isnan(v):
            assert (got & 0x7C00) == 0x7C00 and (got & 0x3FF) != 0
        else:
            assert got == int(rt) == int(rn), (float(v), hex(got), hex(int(rt)))


def _grid_values(prec, emin, emax):
    """All positive finite values of a binary format as exact Fractions, sorted."""
    vals = [Fraction(0)]
    for e in range(emin, emax + 1):
        for m in range(2 ** (prec - 1), 2 ** prec):
            vals.append(Fraction(m) * Fraction(2) ** (e - prec + 1))
    sub = [Fraction(m) * Fraction(2) ** (emin - prec + 1) for m in range(1, 2 ** (prec - 1))]
    return sorted(set(vals + sub))


def _brute_round(x: float, grid, maxf, overflow_at):
    """Nearest-even rounding of the double x onto the grid by exact arithmetic."""
    a = Fraction(abs(x))
    if a >= overflow_at:
        return math.copysign(math.inf, x)
    import bisect
    k = bisect.bisect_left(grid, a)
    if k < len(grid) and grid[k] == a:
        r = grid[k]
    else:
        if k == len(grid):  # above the largest finite value, below the overflow threshold
            return math.copysign(float(maxf), x)
        lo, hi = grid[k - 1], grid[k]
        dl, dh = a - lo, hi - a
        if dl < dh:
            r = lo
        elif dh < dl:
            r = hi
        else:  # tie: the one with an even last significand bit; consecutive
            # grid values alternate in that bit and grid[0] = 0 is even
            r = lo if (k - 1) % 2 == 0 else hi
    return math.copysign(float(r), x)


@pytest.mark.parametrize("fmt", ["bf16", "f16"])
def test_round_from_double_brute_force(fmt):
    if fmt == "bf16":
        prec, emin, emax = 8, -126, 127
        dec = lambda b: oracle.decode("bf16", np.array([b], np.uint16))[0]
        rnd = oracle.round_bf16
    else:
        prec, emin, emax = 11, -14, 15
        dec = lambda b: oracle.decode("f16", np.array([b], np.uint16))[0]
        rnd = oracle.round_f16
    grid = _grid_values(prec, emin, emax)
    maxf = grid[-1]
    ulp_top = Fraction(2) ** (emax - prec + 1)
    overflow_at = maxf + ulp_top / 2  # exactly halfway to 2^(emax+1) rounds to inf (even)
    rng = np.random.default_rng(7)
    xs = []
    # random doubles over the whole range, plus exact midpoints and their neighbours
    xs += list(rng.standard_normal(300) * 10.0 ** rng.integers(-45 if fmt == "bf16" else -9, 38 if fmt == "bf16" else 5, 300))
    idx = rng.integers(1, len(grid) - 1, 300)
    for k in idx:
        mid = (grid[k] + grid[k + 1]) / 2
        m = float(mid)
        xs += [m, np.nextafter(m, 0), np.nextafter(m, np.inf), -m]
    xs += [float(maxf), float(overflow_at), np.nextafter(float(overflow_at), 0), 1e300, -1e300, 5e-324]
    for x in xs:
        x = float(x)
        want = _brute_round(x, grid, maxf, overflow_at)
        got = dec(rnd(x))
        assert _same(float(got), want), (fmt, x, got, want)


def test_round_f32_is_nearest_even():
    rng = np.random.default_rng(3)
    xs = rng.standard_normal(2000) * 10.0 ** rng.integers(-40, 38, 2000)
    for x in xs:
        f = oracle.round_f32(float(x))
        lo = np.nextafter(np.float32(f), np.float32(-np.inf))
        hi = np.nextafter(np.float32(f), np.float32(np.inf))
        e = abs(Fraction(float(f)) - Fraction(float(x)))
        assert e <= abs(Fraction(float(lo)) - Fraction(float(x)))
        assert e <= abs(Fraction(float(hi)) - Fraction(float(x)))
