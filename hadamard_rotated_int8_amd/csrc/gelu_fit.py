"""Coefficients of the GELU epilogue's normal-tail approximation (build-time helper).

The GEMM's GELU epilogue evaluates gelu(y) = y Phi(y) as
    max(y, 0) - |y| h,   h = Phi(-min(|y|, A)) ~ 2^P(t),   t = min(|y|, A) / A in [0, 1],
with P a polynomial of degree DEGREE in t.  Phi(-A) < 1e-9, so clamping |y| at A
changes the result by less than 1e-9 |y|.

What matters is the error of the GELU value, not of log2 h: an error e in P moves
the result by |y| h (2^e - 1) ~ ln2 |y| h e, which is large only where |y| h is
(around |y| ~ 1) and negligible in the far tail.  P is therefore the weighted
minimax fit of log2 Phi(-a) on [0, A] with weight
    w(a) = ln2 Phi(-a) max(a, A0) / max(1, a),
i.e. the error bound |gelu - y Phi(y)| <= max w e max(1, |y|) is spread evenly
over a (the floor A0 keeps the relative error of h small near 0 as well, where
|y| h vanishes).  The fit runs Lawson's iteration: weighted least squares on a
fine grid, reweighting each point by its current error, which converges to the
weighted minimax solution.  Degree 5 reaches 2.4e-7; the float32 evaluation of
common.h stays within 3.3e-7 max(1, |y|) of y Phi(y) (tests/test_gelu_fit.py).

Run `python gelu_fit.py` to print the coefficients that common.h holds.
"""

from __future__ import annotations

import numpy as np
from scipy.special import log_ndtr, ndtr

A = 6.0
A0 = 0.25
DEGREE = 5
POINTS = 120001
ITERATIONS = 300


def weight(a: np.ndarray) -> np.ndarray:
    """GELU error (relative to max(1, |y|)) per unit error of P at |y| = a."""
    return np.log(2.0) * ndtr(-a) * np.maximum(a, A0) / np.maximum(1.0, a)


def fit(degree: int = DEGREE, a_max: float = A):
    """(c[0..degree], weighted max error) with P(t) = sum c[i] t^i ~ log2 Phi(-a), t = a / a_max."""
    a = np.linspace(0.0, a_max, POINTS)
    target = log_ndtr(-a) / np.log(2.0)
    w = weight(a)
    basis = np.vander(a / a_max, degree + 1, increasing=True)
    lw = np.full(a.shape, 1.0 / a.size)
    for _ in range(ITERATIONS):
        sw = np.sqrt(lw) * w
        c = np.linalg.lstsq(basis * sw[:, None], target * sw, rcond=None)[0]
        err = np.abs(basis @ c - target) * w
        lw = lw * err
        lw /= lw.sum()
    return c, float(err.max())


def main() -> None:
    c, err = fit()
    print(f"degree {DEGREE} on [0, {A}]: weighted max error {err:.3e}")
    for i, v in enumerate(c):
        print(f"c{i} = {np.float32(v)!r}  ({v:.17g})")


if __name__ == "__main__":
    main()
