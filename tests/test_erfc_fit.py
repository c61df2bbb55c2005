"""The exact-GeLU kernels' polynomials Q (kErfQ, degree 8, and kErfQ5, degree
5, in mb_device.hpp) are what the committed fit produces, and their fp32
Horner evaluations stay within 2e-7 and 4e-5 relative of 0.5 erfc(x)
exp(z^2/2) / t over the fitted range (scipy's erfcx, independent of the
kernels and of the oracle)."""
import importlib.util
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_elementwise_epilogues_amd", "csrc")


def header_coefficients(name="kErfQ", n=9):
    src = open(os.path.join(CSRC, "mb_device.hpp")).read()
    body = re.search(name + r"\[" + str(n) + r"\]\s*=\s*\{([^}]*)\}", src).group(1)
    return np.array([float(v.strip().rstrip("f")) for v in body.split(",")], np.float32)


def load_fit():
    spec = importlib.util.spec_from_file_location("fit_erfc", os.path.join(CSRC, "fit_erfc.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_header_matches_fit():
    fit = load_fit()
    c = header_coefficients()
    refit = fit.fit()
    assert c.shape == refit.shape == (fit.DEGREE + 1,)
    np.testing.assert_allclose(c, refit, rtol=1e-5, atol=1e-7)


def test_header_polynomial_accuracy():
    fit = load_fit()
    c = header_coefficients()
    t = np.linspace(fit.TMIN, 1.0, 200001)
    rel = np.abs(fit.horner32(c, t) / fit.target(t) - 1.0)
    assert rel.max() < 2e-7, rel.max()
    # Q(1) = 0.5 erfc(0) = 0.5
    assert abs(float(np.sum(c.astype(np.float64))) - 0.5) < 1e-6


def test_half_precision_polynomial_matches_fit_and_accuracy():
    fit = load_fit()
    c = header_coefficients("kErfQ5", 6)
    refit = fit.fit(fit.DEGREE_HALF)
    assert c.shape == refit.shape == (fit.DEGREE_HALF + 1,)
    np.testing.assert_allclose(c, refit, rtol=1e-5, atol=1e-7)
    t = np.linspace(fit.TMIN, 1.0, 200001)
    rel = np.abs(fit.horner32(c, t) / fit.target(t) - 1.0)
    # half of a bf16 ulp is 2^-9, of an fp16 ulp 2^-11 (relative): 4e-5 leaves
    # both outputs within one ulp of the correctly rounded value
    assert rel.max() < 4e-5, rel.max()
