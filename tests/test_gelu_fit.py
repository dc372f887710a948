"""The GEMM's GELU epilogue (gelu_erf in csrc/common.h), checked on the host.

gelu(y) = y Phi(y) is evaluated as max(y, 0) - |y| 2^P(u), u = min(|y|, 6)/3 - 1,
with P the degree-7 fit of log2 Phi(-a) that csrc/gelu_fit.py produces.  These
tests check that the coefficients in common.h are that fit rounded to float32,
and bound the float32 evaluation (fused multiply-adds emulated exactly, the
exponential correctly rounded) against scipy's normal CDF.
"""

import os
import re
import sys

import numpy as np
from scipy.special import ndtr

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "hadamard_rotated_int8_amd", "csrc")


def _kernel_coefficients():
    """c7, c6, ..., c0 as written in gelu_erf (Horner order)."""
    text = open(os.path.join(CSRC, "common.h")).read()
    body = text[text.index("CR_DEVICE float gelu_erf"):]
    body = body[:body.index("\n}\n")]
    first = re.search(r"float p = (-?[0-9.]+)f;", body).group(1)
    rest = re.findall(r"__builtin_fmaf\(p, u, (-?[0-9.]+)f\)", body)
    return [np.float32(float(v)) for v in [first, *rest]]


def _fma32(a, b, c):
    """float32 fused multiply-add: the float64 product of two float32 values is
    exact, the sum is rounded once to float64 and then to float32."""
    return (np.asarray(a, np.float64) * np.asarray(b, np.float64)
            + np.asarray(c, np.float64)).astype(np.float32)


def gelu_kernel(y):
    """gelu_erf's float32 steps: clamp, u, Horner in u, 2^p, final fused multiply-add."""
    y = np.asarray(y, dtype=np.float32)
    cs = _kernel_coefficients()
    a = np.minimum(np.abs(y), np.float32(6.0))
    u = _fma32(a, np.float32(0.33333334), -1.0)
    p = np.full_like(u, cs[0])
    for c in cs[1:]:
        p = _fma32(p, u, c)
    h = np.exp2(p.astype(np.float64)).astype(np.float32)
    return _fma32(-np.abs(y), h, np.maximum(y, np.float32(0.0)))


def test_coefficients_are_the_fit():
    sys.path.insert(0, CSRC)
    try:
        import gelu_fit
    finally:
        sys.path.remove(CSRC)
    fit = gelu_fit.fit()[::-1]  # c7 .. c0
    assert len(fit) == 8
    assert np.array_equal(np.array(_kernel_coefficients()), fit.astype(np.float32))


def test_gelu_error_bound():
    """|gelu_kernel(y) - y Phi(y)| <= 1e-6 max(1, |y|) on a dense grid and at
    large |y| (where the clamp at 6 leaves |y| Phi(-6) < 1e-9 |y| out)."""
    y = np.concatenate([np.linspace(-12.0, 12.0, 2_000_001),
                        np.geomspace(12.0, 1e4, 2000), -np.geomspace(12.0, 1e4, 2000)])
    y32 = y.astype(np.float32)
    exact = y32.astype(np.float64) * ndtr(y32.astype(np.float64))
    got = gelu_kernel(y32).astype(np.float64)
    err = np.abs(got - exact) / np.maximum(1.0, np.abs(y32))
    assert err.max() <= 1e-6, err.max()


def test_gelu_identities():
    """gelu(0) = 0 and gelu(y) - gelu(-y) = y (to float32 rounding)."""
    assert gelu_kernel(np.float32(0.0)) == 0.0
    y = np.linspace(0.01, 8.0, 801).astype(np.float32)
    d = gelu_kernel(y).astype(np.float64) - gelu_kernel(-y).astype(np.float64)
    assert np.max(np.abs(d - y) / y) <= 4e-7
