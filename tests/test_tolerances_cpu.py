"""The parity comparator itself (oracle/tolerances.py): the fp32 rule with a
condition scale passes only what an fp32 evaluation of the exponent can
reach, and no longer lets a tiny value through on an absolute term."""
import numpy as np

from oracle.tolerances import FLOOR_FACTOR, compare


def f32(x):
    return np.asarray(x, np.float32)


def test_absolute_term_hides_a_tiny_wrong_value_without_cond():
    o = f32([-2.3e-7])  # about gelu_tanh(-5)
    k = f32([0.0])      # 100 % off
    ok, st = compare(k, o, o.astype(np.float64), None, "f32")
    assert ok.all() and st["abs_only"] == 1


def test_cond_scaled_rule():
    o64 = np.array([-2.3e-7, 1.0, 3.0e-5])
    o = f32(o64)
    cond = np.array([17.0, 0.0, 5.0])
    # wrong tiny value: refused
    ok, _ = compare(f32([0.0, 1.0, 3.0e-5]), o, o64, None, "f32", cond)
    assert not ok[0] and ok[1] and ok[2]
    # within 8 2^-24 (1 + cond) |o|: passes, counted as floor-only
    k = f32(o64 * (1 + 0.9 * FLOOR_FACTOR * (1 + cond)))
    ok, st = compare(k, o, o64, None, "f32", cond)
    assert ok.all()
    # beyond it: refused
    k = f32(o64 * (1 + 2.0 * FLOOR_FACTOR * (1 + cond)))
    ok, _ = compare(k, o, o64, None, "f32", cond)
    assert not ok[0]


def test_floor_uses_mag_with_cond():
    o64 = np.array([1e-3])
    o = f32(o64)
    mag = np.array([10.0])  # the derivative's summands cancel to 1e-3
    k = f32(o64 + 0.5 * FLOOR_FACTOR * 3.0 * 10.0)
    ok, st = compare(k, o, o64, mag, "f32", np.array([2.0]))
    assert ok.all() and st["floor_only"] == 1
