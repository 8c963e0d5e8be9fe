"""Pins of the oracle's diagonal fallback ("Shampoo -- Second-Order Optimizer", section
"Blocked and distributed variants": a side whose dimension exceeds a threshold drops its
factor and keeps diagonal AdaGrad along it; here the diagonal of the factor as the same
EMA, with the same -1/4 exponent)."""

import numpy as np
import pytest

from oracle import codec
from oracle import shampoo4 as o


def _rng(k):
    return np.random.default_rng([2024, k])


def _orthonormal_columns(rng, m, n):
    return np.linalg.qr(rng.standard_normal((m, n)))[0]


def test_diagonal_statistic_axis_on_rank_one_gradients():
    """G = u v^T: the diagonal of G G^T is u_i^2 |v|^2 (side L sums along a row), that of
    G^T G is v_j^2 |u|^2 (side R sums along a column); a swapped axis fails."""
    rng = _rng(1)
    u, v = rng.standard_normal(5), rng.standard_normal(3)
    G = np.outer(u, v)
    lamL = o.diagonal_statistics(np.zeros(5), o.side_gradient(G, o.SIDE_L), 0.5)
    lamR = o.diagonal_statistics(np.zeros(3), o.side_gradient(G, o.SIDE_R), 0.5)
    b = np.float64(np.float32(0.5))
    assert np.allclose(lamL, (1 - b) * u ** 2 * (v @ v), rtol=1e-14)
    assert np.allclose(lamR, (1 - b) * v ** 2 * (u @ u), rtol=1e-14)
    lam2 = o.diagonal_statistics(lamR, o.side_gradient(G, o.SIDE_R), 0.5)
    assert np.allclose(lam2, b * lamR + (1 - b) * v ** 2 * (u @ u), rtol=1e-14)


@pytest.mark.parametrize("dropped", [o.SIDE_L, o.SIDE_R])
def test_one_sided_equals_two_sided_when_the_dropped_factor_is_diagonal(dropped):
    """Gradients whose dropped-side factor is diagonal at every step (G = Q diag(c) with
    orthonormal columns Q for side R; its transpose for side L) keep that side's 4-bit
    eigenvectors at I in the two-sided method and its eigenvalues equal to the diagonal
    EMA, so both methods give the same codes on the kept side and the same direction."""
    rng = _rng(2 + dropped)
    big, small = 9, 5
    T = 2
    diag = [(dropped == o.SIDE_L, dropped == o.SIDE_R)]
    shape = (small, big) if dropped == o.SIDE_L else (big, small)
    one = o.Shampoo4Oracle([shape], beta=0.9, eps=1e-6, diagonal=diag)
    two = o.Shampoo4Oracle([shape], beta=0.9, eps=1e-6)
    for t in range(1, 6):
        c = 10.0 ** rng.uniform(-1, 1, small)
        G = (_orthonormal_columns(rng, big, small) * c).astype(np.float32)
        if dropped == o.SIDE_L:
            G = np.ascontiguousarray(G.T)
        P1 = one.step([G], t, root_interval=T)[0]
        P2 = two.step([G], t, root_interval=T)[0]
        kept = 1 - dropped
        assert np.array_equal(one.sides[0][kept].codes, two.sides[0][kept].codes)
        d2 = two.sides[0][dropped]
        assert np.array_equal(codec.dequantize_matrix(d2.codes, d2.scales, d2.p),
                              np.eye(d2.p, dtype=np.float32))
        assert np.allclose(one.sides[0][dropped].lam, d2.lam, rtol=1e-6)
        assert np.allclose(P1, P2, rtol=1e-5, atol=1e-6 * np.abs(P2).max()), t


def test_both_sides_diagonal_on_square_diagonal_gradients_is_rmsprop():
    """With both factors dropped, square diagonal gradients give RMSprop without momentum:
    each side's diagonal is the accumulator v <- beta v + (1 - beta) g^2, and
    (v + eps)^(-1/4) twice is (v + eps)^(-1/2)."""
    rng = _rng(4)
    p, beta, eps = 8, 0.95, 1e-6
    orc = o.Shampoo4Oracle([(p, p)], beta=beta, eps=eps, diagonal=[(True, True)])
    v = np.zeros(p, np.float32)
    b32 = np.float32(beta)
    for t in range(1, 7):
        g = (rng.standard_normal(p) * 10.0 ** rng.uniform(-1, 1, p)).astype(np.float32)
        P = orc.step([np.diag(g)], t)[0]
        v = (np.float64(b32) * v + (1.0 - np.float64(b32)) * g.astype(np.float64) ** 2).astype(np.float32)
        upd = g / np.sqrt(v.astype(np.float64) + float(np.float32(eps)))
        assert np.allclose(np.diag(P), upd, rtol=1e-6)
        assert np.count_nonzero(P - np.diag(np.diag(P))) == 0


def test_diagonal_both_sides_general_gradient_closed_form():
    """Both sides diagonal on a general G: P_ij = G_ij (l_i + eps)^(-1/4) (r_j + eps)^(-1/4)
    with l, r the EMAs of the row and column sums of squares."""
    rng = _rng(5)
    m, n, beta, eps = 4, 7, 0.8, 1e-6
    orc = o.Shampoo4Oracle([(m, n)], beta=beta, eps=eps, diagonal=[(True, True)])
    l, r = np.zeros(m), np.zeros(n)
    b = np.float64(np.float32(beta))
    for t in range(1, 4):
        G = rng.standard_normal((m, n)).astype(np.float32)
        P = orc.step([G], t)[0]
        G64 = G.astype(np.float64)
        l = np.float32(b * l + (1 - b) * (G64 ** 2).sum(1)).astype(np.float64)
        r = np.float32(b * r + (1 - b) * (G64 ** 2).sum(0)).astype(np.float64)
        e = np.float64(np.float32(eps))
        dl = np.float32((l + e) ** -0.25).astype(np.float64)
        dr = np.float32((r + e) ** -0.25).astype(np.float64)
        assert np.allclose(P, dl[:, None] * G64 * dr[None, :], rtol=1e-6)


@pytest.mark.parametrize("diag", [(False, True), (True, False), (True, True)])
def test_one_sided_homogeneity(diag):
    """Degree-0 homogeneity survives the fallback (eps = 0, full rank)."""
    rng = _rng(6)
    m, n = 6, 6
    a = o.Shampoo4Oracle([(m, n)], beta=0.9, eps=0.0, diagonal=[diag])
    b = o.Shampoo4Oracle([(m, n)], beta=0.9, eps=0.0, diagonal=[diag])
    for t in range(1, 5):
        G = rng.standard_normal((m, n)).astype(np.float32)
        Pa = a.step([G], t)[0]
        Pb = b.step([np.float32(2) * G], t)[0]
        assert np.linalg.norm(Pa - Pb) <= 1e-6 * np.linalg.norm(Pa)
