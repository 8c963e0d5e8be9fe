"""Quantize the eigenvector matrix or the preconditioner itself (oracle side).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

The abstract of "4-bit Shampoo for Memory-Efficient Network Training" states that
quantizing the preconditioner's eigenvector matrix to 4 bits approximates it far
better than quantizing the preconditioner itself, and that rectifying the quantized
eigenvector matrix's orthogonality also improves the inverse 4th root.  This module
measures that on a given symmetric positive semi-definite factor L, against the
float64 inverse root of the blog's "Computing the inverse fourth root" section
(damping before rooting: (L + eps I)^(-1/4) = U diag((lam + eps)^(-1/4)) U^T):

* ``root_fp32``      U and lam rounded to float32 (the 32-bit state);
* ``root_eigvec4``   U quantized to 4 bits (block-wise linear-square codec, or the
                     dynamic tree codebook the abstract compares it with), then
                     k Bjorck iterations, with the float32 eigenvalues;
* ``root_precond4``  L itself quantized to 4 bits with the same codec (row-major
                     blocks of 64), then the float64 inverse root of the dequantized
                     matrix (symmetrized, eigenvalues clamped at 0 before damping).

Errors are relative Frobenius errors against the float64 truth.  Parity status:
pinned by tests (exact cases: identity and codebook-diagonal factors; float32
rounding bound; Bjorck reduces the 4-bit eigenvector error).
"""

from __future__ import annotations

import numpy as np

from . import codec
from .shampoo4 import bjorck


def eigh_desc(L):
    """Eigenpairs of a symmetric matrix, eigenvalues in descending order (float64)."""
    lam, U = np.linalg.eigh(np.asarray(L, dtype=np.float64))
    order = np.argsort(lam)[::-1]
    return lam[order], U[:, order]


def inverse_root(L, eps: float):
    """(L + eps I)^(-1/4) with eigenvalues clamped at 0 before damping (float64)."""
    lam, U = eigh_desc(0.5 * (np.asarray(L, np.float64) + np.asarray(L, np.float64).T))
    d = (np.maximum(lam, 0.0) + eps) ** -0.25
    return (U * d[None, :]) @ U.T


def root_from(U, lam, eps: float):
    d = (np.maximum(np.asarray(lam, np.float64), 0.0) + eps) ** -0.25
    U = np.asarray(U, np.float64)
    return (U * d[None, :]) @ U.T


def root_fp32(L, eps: float):
    lam, U = eigh_desc(L)
    return root_from(U.astype(np.float32), lam.astype(np.float32), eps)


def root_eigvec4(L, eps: float, bjorck_iters: int = 1, qblock: int = 64,
                 codebook: str = codec.LINEAR_SQUARE):
    lam, U = eigh_desc(L)
    p = U.shape[0]
    codes, scales = codec.quantize_matrix(U.astype(np.float32), qblock, codebook)
    V = bjorck(codec.dequantize_matrix(codes, scales, p, qblock, codebook).astype(np.float64),
               bjorck_iters)
    return root_from(V, lam.astype(np.float32), eps)


def root_precond4(L, eps: float, qblock: int = 64):
    p = np.asarray(L).shape[0]
    codes, scales = codec.quantize_matrix(np.asarray(L, np.float32), qblock)
    L4 = codec.dequantize_matrix(codes, scales, p, qblock).astype(np.float64)
    return inverse_root(L4, eps)


def rel_err(A, B) -> float:
    return float(np.linalg.norm(np.asarray(A) - np.asarray(B)) / np.linalg.norm(np.asarray(B)))


def ablation(L, eps: float, bjorck_iters: int = 1):
    """Relative errors of the inverse 4th root under each storage of the factor."""
    truth = inverse_root(L, eps)
    return {
        "fp32": rel_err(root_fp32(L, eps), truth),
        "eigvec4_no_rectify": rel_err(root_eigvec4(L, eps, 0), truth),
        "eigvec4": rel_err(root_eigvec4(L, eps, bjorck_iters), truth),
        "eigvec4_dt": rel_err(root_eigvec4(L, eps, bjorck_iters, codebook=codec.DYNAMIC_TREE), truth),
        "precond4": rel_err(root_precond4(L, eps), truth),
    }


def ema_factor(gradients, beta: float):
    """L = EMA of G G^T over a gradient sequence (the statistic the step accumulates)."""
    L = None
    for G in gradients:
        G = np.asarray(G, np.float64)
        L = (1.0 - beta) * (G @ G.T) if L is None else beta * L + (1.0 - beta) * (G @ G.T)
    return L
