"""Pins of the ablation oracle (abstract of "4-bit Shampoo for Memory-Efficient Network
Training": quantize the eigenvector matrix rather than the preconditioner, and rectify
it) and the claim itself on synthetic factors."""

import numpy as np
import pytest

from oracle import ablation as ab
from oracle import codec
from workloads import get_workload


def test_identity_is_exact_everywhere():
    L = np.eye(64)
    for k, e in ab.ablation(L, 1e-6).items():
        assert e == 0.0 or e < 1e-15, (k, e)


def test_codebook_diagonal_factor_quantizes_exactly():
    """A diagonal L whose entries are codebook levels times one scale per 64-block row
    quantizes exactly, so the 4-bit preconditioner is exact there (and only there)."""
    lv = codec.LEVELS.astype(np.float64)
    lam = np.abs(lv[[15, 14, 13, 12, 11, 10, 9, 8] * 8])        # 64 positive levels
    L = np.diag(lam)
    root = ab.root_precond4(L, 1e-3)
    assert ab.rel_err(root, ab.inverse_root(L, 1e-3)) < 1e-14


def test_fp32_error_is_float32_rounding():
    rng = np.random.default_rng(0)
    A = rng.standard_normal((96, 96))
    L = A @ A.T
    assert ab.ablation(L, 1e-6)["fp32"] < 2e-6


def test_root_formula_against_scipy():
    import scipy.linalg as sla
    rng = np.random.default_rng(1)
    A = rng.standard_normal((40, 40))
    L = A @ A.T
    want = np.real(sla.fractional_matrix_power(L + 1e-3 * np.eye(40), -0.25))
    assert np.allclose(ab.inverse_root(L, 1e-3), want, rtol=1e-9, atol=1e-12)


@pytest.mark.parametrize("workload", ["single_64x32", "cnn_batch"])
def test_eigenvector_quantization_beats_preconditioner_quantization(workload):
    """The abstract's claim on the workloads' own statistics: the inverse root from 4-bit
    eigenvectors (rectified) is more accurate than from a 4-bit preconditioner, and the
    rectification helps."""
    wl = get_workload(workload)
    b = 0
    L = ab.ema_factor([wl.block_gradient(b, t) for t in range(1, 11)], wl.beta)
    r = ab.ablation(L, 1e-6, 1)
    assert r["eigvec4"] < r["precond4"], r
    assert r["eigvec4"] <= r["eigvec4_no_rectify"], r
    assert r["fp32"] < r["eigvec4"], r
