"""The GEMM's GELU epilogue (gelu_erf in csrc/common.h), checked on the host.

gelu(y) = y Phi(y) is evaluated as max(y, 0) - |y| 2^P(t), t = clamp(|y| / 6, 0, 1),
with P the degree-5 weighted fit of log2 Phi(-a) that csrc/gelu_fit.py produces.
These tests check that the coefficients in common.h are that fit rounded to
float32, and bound the float32 evaluation (multiplies and fused multiply-adds
emulated exactly, the exponential correctly rounded) against scipy's normal CDF.
"""

import os
import re
import sys

import numpy as np
from scipy.special import ndtr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hadamard_rotated_int8_amd", "csrc")


def _kernel_source():
    text = open(os.path.join(CSRC, "common.h")).read()
    body = text[text.index("CR_DEVICE float gelu_erf"):]
    return body[:body.index("\n}\n")]


def _kernel_coefficients():
    """c5, c4, ..., c0 as written in gelu_erf (Horner order)."""
    body = _kernel_source()
    first = re.search(r"float p = (-?[0-9.]+)f;", body).group(1)
    rest = re.findall(r"__builtin_fmaf\(p, t, (-?[0-9.]+)f\)", body)
    return [np.float32(float(v)) for v in [first, *rest]]


def _kernel_inv6():
    return np.float32(float(re.search(r"fabsf\(y\) \* ([0-9.]+)f", _kernel_source()).group(1)))


def _fma32(a, b, c):
    """float32 fused multiply-add: the float64 product of two float32 values is
    exact, the sum is rounded once to float64 and then to float32."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)
            + np.asarray(c, np.float64)).astype(np.float32)


def gelu_kernel(y):
    """gelu_erf's float32 steps: t (one rounded multiply, clamped), Horner in t,
    2^p, final fused multiply-add."""
    y = np.asarray(y, dtype=np.float32)
    cs = _kernel_coefficients()
    t = np.clip((np.abs(y).astype(np.float64) * np.float64(_kernel_inv6())).astype(np.float32),
                np.float32(0.0), np.float32(1.0))
    p = np.full_like(t, cs[0])
    for c in cs[1:]:
        p = _fma32(p, t, c)
    h = np.exp2(p.astype(np.float64)).astype(np.float32)
    return _fma32(-np.abs(y), h, np.maximum(y, np.float32(0.0)))


def test_coefficients_are_the_fit():
    sys.path.insert(0, CSRC)
    try:
        import gelu_fit
    finally:
        sys.path.remove(CSRC)
    fit, err = gelu_fit.fit()
    fit = fit[::-1]  # c5 .. c0
    assert len(fit) == 6 and err < 3e-7
    assert _kernel_inv6() == np.float32(1.0 / gelu_fit.A)
    # the float32 rounding of the fit (to one unit in the last place, so that
    # the check does not hinge on the last bits of the host's least squares)
    k = np.array(_kernel_coefficients())
    f = fit.astype(np.float32)
    assert np.all(np.abs(k - f) <= np.spacing(np.abs(f))), (k, f)


def test_gelu_error_bound():
    """|gelu_kernel(y) - y Phi(y)| <= 4e-7 max(1, |y|) on a dense grid, near 0
    and at large |y| (where the clamp at 6 leaves |y| Phi(-6) < 1e-9 |y| out)."""
    y = np.concatenate([np.linspace(-12.0, 12.0, 2_000_001),
                        np.geomspace(12.0, 1e4, 2000), -np.geomspace(12.0, 1e4, 2000),
                        np.geomspace(1e-8, 1e-2, 2000), -np.geomspace(1e-8, 1e-2, 2000)])
    y32 = y.astype(np.float32)
    exact = y32.astype(np.float64) * ndtr(y32.astype(np.float64))
    got = gelu_kernel(y32).astype(np.float64)
    err = np.abs(got - exact) / np.maximum(1.0, np.abs(y32))
    assert err.max() <= 4e-7, err.max()
    # near 0 the relative error stays small too (the weight's floor)
    small = (np.abs(y32) < 1e-2) & (y32 != 0)
    rel = np.abs(got - exact)[small] / np.abs(exact[small])
    assert rel.max() <= 5e-6, rel.max()


def test_gelu_identities():
    """gelu(0) = 0, gelu(y) - gelu(-y) = y (to float32 rounding), and the sign of
    gelu(y) is that of y."""
    assert gelu_kernel(np.float32(0.0)) == 0.0
    y = np.linspace(0.01, 8.0, 801).astype(np.float32)
    d = gelu_kernel(y).astype(np.float64) - gelu_kernel(-y).astype(np.float64)
    assert np.max(np.abs(d - y) / y) <= 4e-7
    assert np.all(gelu_kernel(y) > 0) and np.all(gelu_kernel(-y) <= 0)
