"""Pins of the grafting oracle ("Shampoo -- Second-Order Optimizer", section "Grafting:
borrow a step size that already works") against closed forms: the step carries the
grafted method's norm and Shampoo's direction; Adam's direction is known exactly at the
first step and under a constant gradient."""

import numpy as np
import pytest

from oracle import graft


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


@pytest.mark.parametrize("mode", [graft.SGD, graft.ADAM])
def test_step_norm_is_the_grafted_norm(mode):
    """With eps_graft = 0 the step has exactly eta * ||d_graft||_F and the direction of P."""
    W, G, P = _rand((7, 5), 1), _rand((7, 5), 2), _rand((7, 5), 3)
    lr = 0.37
    Wn, m, v, s = graft.graft_step(W, G, P, mode=mode, lr=lr, eps_graft=0.0, t=1)
    step = W - Wn
    if mode == graft.SGD:
        d_graft = G
    else:
        d_graft = G / (np.abs(G) + 1e-8)          # first Adam step, worked by hand
    assert np.isclose(np.linalg.norm(step), lr * np.linalg.norm(d_graft), rtol=1e-12)
    # same direction as P, with a positive factor (W moves against P)
    c = np.sum(step * P) / np.sum(P * P)
    assert c > 0 and np.allclose(step, c * P, rtol=0, atol=1e-12)


def test_direction_scale_invariance():
    """Rescaling d_shampoo by c > 0 leaves the grafted step unchanged (eps_graft = 0)."""
    W, G, P = _rand((6, 9), 4), _rand((6, 9), 5), _rand((6, 9), 6)
    a = graft.graft_step(W, G, P, mode=graft.SGD, lr=0.1, eps_graft=0.0)[0]
    b = graft.graft_step(W, G, 1e3 * P, mode=graft.SGD, lr=0.1, eps_graft=0.0)[0]
    assert np.allclose(a, b, rtol=1e-12, atol=1e-14)


def test_sgd_graft_closed_form():
    W, G, P = _rand((4, 3), 7), _rand((4, 3), 8), _rand((4, 3), 9)
    eps = 1e-3
    Wn, m, v, s = graft.graft_step(W, G, P, mode=graft.SGD, lr=2.0, eps_graft=eps)
    want = W - 2.0 * np.sqrt(np.sum(G * G)) / (np.sqrt(np.sum(P * P)) + eps) * P
    assert m is None and v is None
    assert np.allclose(Wn, want, rtol=1e-13, atol=0)


def test_adam_first_step_is_sign_of_gradient():
    """t = 1: m_hat = g and v_hat = g^2, so with eps_adam = 0 the direction is sign(g)."""
    g = _rand((5, 5), 10)
    g[0, 0] = 0.5
    m, v = graft.adam_moments(np.zeros_like(g), np.zeros_like(g), g, 0.9, 0.999)
    assert np.allclose(m, 0.1 * g, rtol=1e-15) and np.allclose(v, 0.001 * g * g, rtol=1e-12)
    d = graft.adam_direction(m, v, 1, 0.9, 0.999, 0.0)
    assert np.allclose(d, np.sign(g), rtol=1e-12, atol=0)


@pytest.mark.parametrize("t_end", [2, 5, 40])
def test_adam_constant_gradient_keeps_unit_direction(t_end):
    """Under a constant gradient the bias correction undoes the moments' zero start
    exactly: m_hat = g and v_hat = g^2 at every step, so the direction stays
    g / (|g| + eps_adam).  A wrong correction exponent or a dropped (1 - beta) fails."""
    g = _rand((3, 4), 11)
    beta1, beta2, eps_a = 0.8, 0.95, 1e-3
    W = np.zeros_like(g)
    P = _rand((3, 4), 12)
    m = v = None
    for t in range(1, t_end + 1):
        Wn, m, v, s = graft.graft_step(W, g, P, mode=graft.ADAM, lr=1.0, eps_graft=0.0, t=t,
                                       m=m, v=v, beta1=beta1, beta2=beta2, eps_adam=eps_a)
    d = graft.adam_direction(m, v, t_end, beta1, beta2, eps_a)
    assert np.allclose(d, g / (np.abs(g) + eps_a), rtol=1e-10, atol=0)
    assert np.isclose(s, np.linalg.norm(g / (np.abs(g) + eps_a)) / np.linalg.norm(P), rtol=1e-10)


def test_zero_direction_gives_no_step():
    W, G = _rand((3, 3), 13), _rand((3, 3), 14)
    Wn, _, _, s = graft.graft_step(W, G, np.zeros((3, 3)), mode=graft.SGD, lr=1.0, eps_graft=1e-6)
    assert np.array_equal(Wn, W)
