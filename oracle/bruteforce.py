"""Full-matrix constructions used only to pin the oracle on tiny sizes.

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "Shampoo -- Second-Order Optimizer", sections "The full-matrix ideal"
(H = sum of vec(g) vec(g)^T over steps) and "Where the fourth root comes from"
(column-major vec with (A kron B) vec(X) = vec(B X A^T); the Kronecker bound
relating H to R^(1/2) kron L^(1/2); (R^(1/2) kron L^(1/2))^(-1/2) acting on
vec(G) as L^(-1/4) G R^(-1/4)).

These routines go through the mn x mn matrices explicitly, with SciPy's
general matrix functions (Schur-based ``sqrtm`` and
``fractional_matrix_power``), so they share no route with the eigen form the
oracle uses.
"""

from __future__ import annotations

import numpy as np
import scipy.linalg as sla


def vec(X) -> np.ndarray:
    """Column-major vectorization (stack the columns)."""
    return np.asarray(X, dtype=np.float64).reshape(-1, order="F")


def unvec(x, m: int, n: int) -> np.ndarray:
    return np.asarray(x, dtype=np.float64).reshape((m, n), order="F")


def full_adagrad_statistic(Gs) -> np.ndarray:
    """H = sum_s vec(G_s) vec(G_s)^T, an (mn x mn) matrix."""
    H = None
    for G in Gs:
        g = vec(G)
        H = np.outer(g, g) if H is None else H + np.outer(g, g)
    return H


def psd_sqrt(A) -> np.ndarray:
    """Principal square root of a symmetric PSD matrix via SciPy's Schur route."""
    S = sla.sqrtm(np.asarray(A, dtype=np.float64))
    S = np.real(S)
    return 0.5 * (S + S.T)


def kronecker_root_direction(L, R, G) -> np.ndarray:
    """Apply (R^(1/2) kron L^(1/2))^(-1/2) to vec(G) and reshape to [m, n].

    The mn x mn matrix is formed explicitly and its inverse square root taken
    with ``scipy.linalg.fractional_matrix_power``.
    """
    G = np.asarray(G, dtype=np.float64)
    m, n = G.shape
    K = np.kron(psd_sqrt(R), psd_sqrt(L))
    K = 0.5 * (K + K.T)
    Kinv_half = np.real(sla.fractional_matrix_power(K, -0.5))
    return unvec(Kinv_half @ vec(G), m, n)


def full_matrix_adagrad_direction(Gs, eps: float) -> np.ndarray:
    """(H + eps I)^(-1/2) vec(G_last), the full-matrix ideal, reshaped."""
    G = np.asarray(Gs[-1], dtype=np.float64)
    m, n = G.shape
    H = full_adagrad_statistic(Gs)
    M = H + eps * np.eye(H.shape[0])
    Minv_half = np.real(sla.fractional_matrix_power(M, -0.5))
    return unvec(Minv_half @ vec(G), m, n)
