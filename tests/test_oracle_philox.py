"""Pins for the oracle's dropout RNG: Philox4x32-10 and the keep mask.

The block function is checked word for word against two independent
installed implementations, compiled here as host programs from their
headers: rocRAND's ``philox4x32_10_engine`` and ATen's ``philox_engine``.
Under the mask layout (counter = (element/4, offset), key = seed, word
element mod 4) an element's word is word (i mod 4) of rocRAND's
engine(seed, subsequence=offset, offset=4*(i/4)), i.e. ATen's
engine(seed, subsequence=offset, offset=i/4).
"""
import math
import os
import subprocess
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle

PINS = os.path.join(os.path.dirname(os.path.abspath(__file__)), "pins")
M64 = (1 << 64) - 1


@pytest.fixture(scope="module")
def engines(tmp_path_factory):
    d = tmp_path_factory.mktemp("philox_pins")
    exe = {}
    rocrand_inc = "/opt/rocm/include"
    if not os.path.exists(os.path.join(rocrand_inc, "rocrand", "rocrand_philox4x32_10.h")):
        pytest.skip("rocRAND headers not installed")
    torch_inc = os.path.join(os.path.dirname(torch.__file__), "include")
    builds = {
        "rocrand": ["g++", "-O1", "-std=c++17", "-D__HIP_PLATFORM_AMD__", "-I" + rocrand_inc,
                    os.path.join(PINS, "philox_rocrand.cpp"), "-o", str(d / "pr")],
        "aten": ["g++", "-O1", "-std=c++17", "-I" + torch_inc, os.path.join(PINS, "philox_aten.cpp"),
                 "-o", str(d / "pa")],
    }
    for name, cmd in builds.items():
        subprocess.run(cmd, check=True)
        exe[name] = cmd[-1]
    return exe


def _blocks(exe, seed, sub, q0, count):
    out = subprocess.run([exe, str(seed), str(sub), str(q0), str(count)], check=True,
                         capture_output=True, text=True).stdout.split("\n")
    return [[int(w) for w in line.split()] for line in out if line.strip()]


CASES = [
    (0, 0, 0),
    (1234, 0, 0),
    (5001, 0, 0),
    (5002, 0, 0),
    (M64, M64, 2**40 + 7),
    (0xDEADBEEFCAFEF00D, 1, 2**32 - 2),
    (42, 2**32, 12345),
    (2**63 + 11, 2**63 + 5, 2**61 + 3),  # rocRAND takes the word offset 4q as 64-bit
]


@pytest.mark.parametrize("seed,sub,q0", CASES)
def test_block_function_matches_rocrand_and_aten(engines, seed, sub, q0):
    n = 16
    ref_r = _blocks(engines["rocrand"], seed, sub, q0, n)
    ref_a = _blocks(engines["aten"], seed, sub, q0, n)
    for k in range(n):
        q = q0 + k
        ctr = [q & 0xFFFFFFFF, (q >> 32) & 0xFFFFFFFF, sub & 0xFFFFFFFF, (sub >> 32) & 0xFFFFFFFF]
        key = [seed & 0xFFFFFFFF, (seed >> 32) & 0xFFFFFFFF]
        got = oracle.philox4x32_10(ctr, key)
        assert got == ref_r[k] == ref_a[k], (seed, sub, q, got, ref_r[k], ref_a[k])


@pytest.mark.parametrize("p", [0.0, 2.0**-32, 0.1, 0.5, 1 - 2.0**-24, 1.0])
def test_threshold_is_floor_of_float_p_times_2_32(p):
    pf = np.float32(p)
    want = min(math.floor(Fraction(float(pf)) * 2**32), 2**32)
    assert oracle.drop_threshold(float(pf)) == want
    if pf < 1:
        assert oracle.keep_scale(float(pf)) == float(np.float32(1.0 / (1.0 - float(pf))))


def test_float_p_01_threshold_value():
    # the dtype of p is part of the contract: float 0.1 is 0.10000000149...
    assert oracle.drop_threshold(0.1) == 429496736


@pytest.mark.parametrize("p", [0.0, 2.0**-32, 0.1, 0.5, 1 - 2.0**-24, 1.0])
@pytest.mark.parametrize("offset", [0, 1, 2**32])
@pytest.mark.parametrize("row0", [0, 3])
def test_mask_bits_brute_force_4x8(engines, p, offset, row0):
    """Every bit of a 4x8 mask against a direct rocRAND call for that element."""
    T, H, seed = 4, 8, 1234
    bits = oracle.dropout_mask(T, H, p, seed, offset, row0)
    theta = min(math.floor(Fraction(float(np.float32(p))) * 2**32), 2**32)
    g0 = row0 * H
    blocks = _blocks(engines["rocrand"], seed, offset, g0 // 4, (T * H + 3) // 4 + 1)
    for t in range(T):
        for j in range(H):
            loc = t * H + j
            gi = (row0 + t) * H + j
            word = blocks[gi // 4 - g0 // 4][gi % 4]
            want = int(word >= theta)
            assert (bits[loc >> 3] >> (loc & 7)) & 1 == want, (t, j, p, offset)


def test_mask_tail_byte_is_zero_padded():
    bits = oracle.dropout_mask(3, 5, 0.0, 1, 0)  # 15 elements, all kept
    assert len(bits) == 2 and bits[0] == 0xFF and bits[1] == 0x7F


@pytest.mark.parametrize("p", [0.1, 0.5, 0.9])
def test_kept_fraction_within_3_sigma(p):
    T, H = 256, 4096
    bits = oracle.dropout_mask(T, H, p, 1234, 0)
    n = T * H
    kept = int(np.unpackbits(bits, bitorder="little")[:n].sum())
    sigma = math.sqrt(p * (1 - p) / n)
    assert abs(kept / n - (1 - p)) <= 3 * sigma


def test_offsets_give_independent_masks():
    T, H, p = 128, 1024, 0.5
    a = np.unpackbits(oracle.dropout_mask(T, H, p, 99, 0), bitorder="little")
    b = np.unpackbits(oracle.dropout_mask(T, H, p, 99, 1), bitorder="little")
    c = np.unpackbits(oracle.dropout_mask(T, H, p, 100, 0), bitorder="little")
    n = T * H
    for other in (b, c):
        both = float((a & other).sum()) / n
        assert abs(both - 0.25) < 4 * math.sqrt(0.25 * 0.75 / n)


def test_word_bits_are_balanced():
    # every bit position of the generated words is set about half the time
    words = []
    for q in range(4096):
        words += oracle.philox4x32_10([q, 0, 0, 0], [1234, 0])
    w = np.array(words, dtype=np.uint64)
    n = len(words)
    for b in range(32):
        frac = float(((w >> b) & 1).sum()) / n
        assert abs(frac - 0.5) < 5 * math.sqrt(0.25 / n)
