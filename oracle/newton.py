"""Coupled Newton iteration for the inverse p-th root (oracle side).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "Shampoo -- Second-Order Optimizer" (aicassindra.com), section "Computing the
inverse fourth root", second route: using matrix products only, scale A so that its
norm is at most 1, start from X = I and M = A, and repeat
    F = ((p + 1) I - M) / p,   X <- X F,   M <- F^p M;
M tends to I and X to A^(-1/p), quadratically once M is close to I.

Readings: the damping of the same section's first route is applied first (A = L + eps I,
so the result is (L + eps I)^(-1/p)); the norm used for the scaling is the Frobenius
norm c = ||A||_F (an upper bound of the spectral norm), and the root of the original
matrix is c^(-1/p) times the root of A / c; the iteration count is fixed by the caller.

Float64 throughout; parity status: pinned by tests (diagonal closed form, the invariant
M = X^p A / c at every iteration, agreement with the eigendecomposition route).
"""

from __future__ import annotations

import numpy as np


def coupled_newton_inverse_root(L, eps: float, iters: int, p: int = 4, return_state: bool = False):
    """(L + eps I)^(-1/p) by the coupled Newton iteration, float64."""
    L = np.asarray(L, dtype=np.float64)
    n = L.shape[0]
    I = np.eye(n)
    A = L + eps * I
    c = float(np.linalg.norm(A))
    M = A / c
    X = I.copy()
    for _ in range(iters):
        F = ((p + 1) * I - M) / p
        X = X @ F
        M = np.linalg.matrix_power(F, p) @ M
    out = X * c ** (-1.0 / p)
    if return_state:
        return out, X, M, c
    return out
