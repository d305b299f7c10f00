"""The software 2^x used by fa_fwd_variant 3: the constants in common.h are the ones the
committed fit produces, and the float32 evaluation, done here step by step as the kernel
does it, stays within 1e-4 relative of the exact 2^x over the range the softmax uses."""
import importlib.util
import os
import re

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_tiled_attention_36_amd", "csrc")


def kernel_coefficients():
    src = open(os.path.join(CSRC, "common.h")).read()
    body = src[src.index("float poly_exp2(float x)"):]
    body = body[:body.index("}")]
    return [float(x) for x in re.findall(r"([0-9]+\.[0-9]+)f", body) if float(x) < 1.5]


def test_constants_match_the_fit():
    spec = importlib.util.spec_from_file_location("fit", os.path.join(CSRC, "fit_exp2_poly.py"))
    fit = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(fit)
    c, err = fit.fit()
    c3, c2, c1, c0 = kernel_coefficients()[:4]   # Horner order in the kernel
    np.testing.assert_allclose([c0, c1, c2, c3], c, rtol=1e-7)
    assert err < 1e-4


def test_float32_evaluation_error():
    c3, c2, c1, c0 = (np.float32(x) for x in kernel_coefficients()[:4])
    x = np.linspace(-60.0, 0.0, 200001).astype(np.float32)     # x = s*log2e - m <= 0
    xc = np.maximum(x, np.float32(-200.0))
    n = np.rint(xc).astype(np.float32)
    f = (xc - n).astype(np.float32)
    p = np.float32(c3) * f + c2
    p = (p * f + c1).astype(np.float32)
    p = (p * f + c0).astype(np.float32)
    y = np.ldexp(p, n.astype(np.int32))
    rel = np.abs(y.astype(np.float64) - np.exp2(x.astype(np.float64))) / np.exp2(x.astype(np.float64))
    assert rel.max() < 1e-4
    # a masked score (-inf) gives exactly 0
    xm = np.maximum(np.float32(-np.inf), np.float32(-200.0))
    assert np.ldexp(np.float32(1.0), int(np.rint(xm))) == 0.0
