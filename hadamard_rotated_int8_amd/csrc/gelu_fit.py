"""Coefficients of the GELU epilogue's normal-tail approximation (build-time helper).

The GEMM's GELU epilogue evaluates gelu(y) = y Phi(y) as
    max(y, 0) - |y| h(min(|y|, A)),   h(a) = Phi(-a),
with h(a) = 2^P(u), u = 2 a / A - 1 in [-1, 1], and P a polynomial of degree
DEGREE fitted to log2 Phi(-a) by least squares at Chebyshev nodes (close to the
minimax fit), then written in powers of u for Horner's rule.  Phi(-A) < 1e-9,
so clamping |y| at A changes the result by less than 1e-9 |y|.

Run `python gelu_fit.py` to print the coefficients that common.h holds and the
fit's error over a fine grid; tests/test_gelu_fit.py checks the committed
coefficients (rounded to float32, evaluated in float32 as the kernel does)
against scipy's normal CDF.
"""

from __future__ import annotations

import numpy as np
from scipy.special import log_ndtr

A = 6.0
DEGREE = 7
NODES = 4000


def fit(degree: int = DEGREE, a_max: float = A) -> np.ndarray:
    """Monomial coefficients c[0..degree] of P(u) ~ log2 Phi(-a), u = 2a/A - 1."""
    k = np.arange(NODES)
    u = np.cos(np.pi * (k + 0.5) / NODES)  # Chebyshev nodes in [-1, 1]
    a = (u + 1.0) * a_max / 2.0
    cheb = np.polynomial.chebyshev.chebfit(u, log_ndtr(-a) / np.log(2.0), degree)
    return np.polynomial.chebyshev.cheb2poly(cheb)


def main() -> None:
    c = fit()
    a = np.linspace(0.0, A, 600001)
    u = 2.0 * a / A - 1.0
    p = np.polynomial.polynomial.polyval(u, c)
    err = np.abs(p - log_ndtr(-a) / np.log(2.0))
    print(f"degree {DEGREE} on [0, {A}]: max |P - log2 Phi(-a)| = {err.max():.3e}")
    for i, v in enumerate(c):
        print(f"c{i} = {np.float32(v)!r}  ({v:.17g})")


if __name__ == "__main__":
    main()
