"""The exact-GeLU kernels' polynomial Q (kErfQ in mb_device.hpp) is what the
committed fit produces, and its fp32 Horner evaluation stays within 2e-7
relative of 0.5 erfc(x) exp(z^2/2) / t over the fitted range (scipy's erfcx,
independent of the kernels and of the oracle)."""
import importlib.util
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_elementwise_epilogues_amd", "csrc")


def header_coefficients():
    src = open(os.path.join(CSRC, "mb_device.hpp")).read()
    body = re.search(r"kErfQ\[9\]\s*=\s*\{([^}]*)\}", src).group(1)
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
