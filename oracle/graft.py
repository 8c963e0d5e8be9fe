"""Grafting and the weight update after the preconditioner (oracle side).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "Shampoo -- Second-Order Optimizer" (aicassindra.com), section
"Grafting: borrow a step size that already works".  The page takes the step's
direction from Shampoo, d_shampoo = L^(-1/4) G R^(-1/4), and its Frobenius norm,
per layer or per block, from the step another optimizer (Adam or SGD) would
have taken, d_graft:

    step = eta * ||d_graft||_F / (||d_shampoo||_F + eps) * d_shampoo
    W   <- W - step

Readings (the page names the grafted methods but does not write them out):

* per block: the norms are taken over one block G:[m, n], the unit the library
  preconditions;
* SGD graft: d_graft = G (the plain gradient step before its learning rate,
  which eta carries);
* Adam graft: d_graft = m_hat / (sqrt(v_hat) + eps_adam), Adam's update
  direction as published by Kingma and Ba ("Adam: A method for stochastic
  optimization", in the reference list of the ICCV 2025 record of the 4-bit
  preconditioned-optimization paper): per element, with the gradient g at step
  t = 1, 2, ...,
      m <- beta1 m + (1 - beta1) g,     v <- beta2 v + (1 - beta2) g^2,
      m_hat = m / (1 - beta1^t),        v_hat = v / (1 - beta2^t);
  the moments start at zero and are updated by the same call.

Float64 throughout; parity status: pinned by tests (norm matching, scale
invariance of the direction, Adam's first step and constant-gradient steps in
closed form, zero-direction guard).
"""

from __future__ import annotations

import numpy as np

SGD = 0
ADAM = 1


def adam_moments(m, v, g, beta1: float, beta2: float):
    """One Adam moment update (elementwise, float64)."""
    g = np.asarray(g, dtype=np.float64)
    m = beta1 * np.asarray(m, dtype=np.float64) + (1.0 - beta1) * g
    v = beta2 * np.asarray(v, dtype=np.float64) + (1.0 - beta2) * g * g
    return m, v


def adam_direction(m, v, t: int, beta1: float, beta2: float, eps_adam: float):
    """Bias-corrected Adam direction m_hat / (sqrt(v_hat) + eps_adam)."""
    m_hat = m / (1.0 - beta1 ** t)
    v_hat = v / (1.0 - beta2 ** t)
    return m_hat / (np.sqrt(v_hat) + eps_adam)


def graft_scale(d_graft, d_shampoo, eps_graft: float) -> float:
    """||d_graft||_F / (||d_shampoo||_F + eps_graft)."""
    return float(np.linalg.norm(np.asarray(d_graft, np.float64)) /
                 (np.linalg.norm(np.asarray(d_shampoo, np.float64)) + eps_graft))


def graft_step(W, G, P, *, mode: int, lr: float, eps_graft: float, t: int = 1,
               m=None, v=None, beta1: float = 0.9, beta2: float = 0.999, eps_adam: float = 1e-8):
    """Grafted update of one block.

    W, G, P: [m, n] weights, gradient and preconditioned gradient d_shampoo.
    Returns (W_new, m_new, v_new, scale) with m_new, v_new None for SGD.
    """
    W = np.asarray(W, dtype=np.float64)
    G = np.asarray(G, dtype=np.float64)
    P = np.asarray(P, dtype=np.float64)
    if mode == SGD:
        d_graft = G
        m_new = v_new = None
    elif mode == ADAM:
        m0 = np.zeros_like(G) if m is None else m
        v0 = np.zeros_like(G) if v is None else v
        m_new, v_new = adam_moments(m0, v0, G, beta1, beta2)
        d_graft = adam_direction(m_new, v_new, t, beta1, beta2, eps_adam)
    else:
        raise ValueError("mode must be SGD or ADAM")
    s = graft_scale(d_graft, P, eps_graft)
    return W - lr * s * P, m_new, v_new, s
