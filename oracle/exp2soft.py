"""Software base-2 exponential for part of the softmax exponentials (float32 emulation).

Test infrastructure only (see the package docstring).

[HW] section 0x09 moves a fraction of the exp2 evaluations of the softmax off the
exponential unit onto the FMA pipe: a Cody-Waite style range reduction x = n + f with
an integer n and f in [0, 1), a low-degree polynomial for 2^f, and the result scaled by
2^n through the exponent.  The page prints its own degree-3 coefficients and quotes
their float32 maximum relative error (8.77e-5); those numbers are a comparison point
only.  This module derives its own coefficients: the degree-3 polynomial minimising
the maximum *relative* error of 2^f on [0, 1], found by the Remez exchange (solve for
the polynomial that equioscillates on deg + 2 reference points, move the references
to the error's extrema, repeat).

``soft_exp2_f32`` states exactly what a float32 implementation computes:
    x' = max(x, -150)                  (so that -inf and deep underflow give 0)
    n  = floor(x'),  f = x' - n        (exact in float32)
    p  = ((c3 f + c2) f + c1) f + c0   (three fused multiply-adds, Horner order)
    y  = p * 2^n                       (exact scaling; 0 below the float32 range)
"""
from __future__ import annotations

import numpy as np

DEGREE = 3


def fit_coefficients(degree: int = DEGREE, iters: int = 40, grid_points: int = 200001):
    """Minimax relative-error polynomial for 2^f on [0, 1]: (coefficients c0..c_deg in
    float64, maximum relative error on the grid)."""
    n = degree + 2
    refs = 0.5 - 0.5 * np.cos(np.pi * np.arange(n) / (n - 1))     # Chebyshev extrema
    grid = np.linspace(0.0, 1.0, grid_points)
    target = np.exp2(grid)
    coef = None
    for _ in range(iters):
        # p(x_i) - 2^x_i = (-1)^i E 2^x_i  at the references
        A = np.zeros((n, n))
        for i, x in enumerate(refs):
            A[i, :degree + 1] = x ** np.arange(degree + 1)
            A[i, degree + 1] = -((-1.0) ** i) * np.exp2(x)
        sol = np.linalg.solve(A, np.exp2(refs))
        coef = sol[:degree + 1]
        err = (np.polyval(coef[::-1], grid) - target) / target
        # new references: the endpoints and the interior extrema of the error
        d = np.diff(err)
        interior = np.nonzero(d[:-1] * d[1:] < 0)[0] + 1
        idx = np.concatenate([[0], interior, [grid_points - 1]])
        if len(idx) != n:
            break
        refs = grid[idx]
    err = (np.polyval(coef[::-1], grid) - target) / target
    return coef, float(np.max(np.abs(err)))


def coefficients_f32():
    """The fitted coefficients rounded to float32 (c0, c1, c2, c3)."""
    coef, _ = fit_coefficients()
    return tuple(np.float32(c) for c in coef)


def _fma_f32(a, b, c):
    # a * b is exact in float64 for float32 operands; one rounding of the sum to
    # float64 and one to float32 (a correctly rounded fma can differ by 1 ulp in rare
    # double-rounding cases, which the tests allow)
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(np.float32)


def soft_exp2_f32(x):
    """The software exp2 of the module docstring, in float32 arithmetic."""
    c0, c1, c2, c3 = coefficients_f32()
    x = np.maximum(np.asarray(x, dtype=np.float32), np.float32(-150.0))
    n = np.floor(x)
    f = (x - n).astype(np.float32)
    p = _fma_f32(np.full_like(f, c3), f, np.full_like(f, c2))
    p = _fma_f32(p, f, np.full_like(f, c1))
    p = _fma_f32(p, f, np.full_like(f, c0))
    return np.ldexp(p, n.astype(np.int32)).astype(np.float32)
