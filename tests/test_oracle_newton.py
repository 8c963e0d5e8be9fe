"""Pins of the coupled Newton inverse-root oracle ("Shampoo -- Second-Order Optimizer",
section "Computing the inverse fourth root", the matrix-multiply route)."""

import numpy as np
import pytest

from oracle import ablation as ab
from oracle import newton as nw


def test_diagonal_closed_form():
    a = np.array([1e-3, 0.1, 1.0, 7.0, 300.0])
    X = nw.coupled_newton_inverse_root(np.diag(a), 1e-4, 40)
    assert np.allclose(X, np.diag((a + 1e-4) ** -0.25), rtol=1e-12, atol=0)


@pytest.mark.parametrize("iters", [1, 3, 8])
def test_invariant_m_equals_x4_a_over_c(iters):
    """The coupled update keeps M = X^p (A / c) at every iteration (all iterates are
    polynomials in A and commute); a wrong update order or power breaks it."""
    rng = np.random.default_rng(2)
    B = rng.standard_normal((20, 20))
    L = B @ B.T
    _, X, M, c = nw.coupled_newton_inverse_root(L, 1e-2, iters, return_state=True)
    A = (L + 1e-2 * np.eye(20)) / c
    assert np.allclose(M, np.linalg.matrix_power(X, 4) @ A, rtol=0, atol=1e-11)


def test_agrees_with_eigendecomposition_route():
    rng = np.random.default_rng(3)
    B = rng.standard_normal((48, 48))
    L = B @ B.T / 48
    X = nw.coupled_newton_inverse_root(L, 1e-3, 30)
    assert ab.rel_err(X, ab.inverse_root(L, 1e-3)) < 1e-12
    # and the fourth power inverts the damped factor
    assert np.allclose(np.linalg.matrix_power(X, 4) @ (L + 1e-3 * np.eye(48)), np.eye(48), atol=1e-10)


def test_square_root_variant_p2():
    """p = 2 gives the inverse square root (same iteration, another p)."""
    a = np.array([0.5, 2.0, 9.0])
    X = nw.coupled_newton_inverse_root(np.diag(a), 0.0, 40, p=2)
    assert np.allclose(X, np.diag(a ** -0.5), rtol=1e-12)
