"""4-bit Shampoo preconditioner step, plain float64 NumPy (oracle side).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

For one weight block G:[m, n] the method keeps two Kronecker factors: the
row-space factor L:[m, m] (side "L") and the column-space factor R:[n, n]
(side "R").  ("Shampoo -- Second-Order Optimizer", section "Kronecker
factorization".)  Following the abstract of "4-bit Shampoo for
Memory-Efficient Network Training", a factor is never stored as a matrix: it
is stored as its eigenvector matrix U (4-bit codes, see ``codec``) and its
eigenvalues (float32).

Per side X with order p the state is
    codes, scales   4-bit eigenvector matrix U (p x p, eigenvectors = columns)
    lam             float32 eigenvalues, >= 0
    root_codes, root_scales, d   the root snapshot: eigenvectors and the
                    float32 root scaling d_i = (lam_i + eps)^(-1/4)

The step, in the order the method describes it (section references are to
the Shampoo blog page unless the abstract is named):

update_stats(G)  (side R uses G^T where side L uses G)
  1. V~ = dequantize(codes, scales)                                 [abstract]
  2. Bjorck rectification, k times: V <- 1.5 V - 0.5 V (V^T V)      [abstract]
  3. Statistics as an exponential moving average
        L~ = beta * V diag(lam) V^T + (1 - beta) * G G^T
     ("Kronecker factorization" for G G^T; "Pitfalls" for the EMA)
  4. Eigen refresh warm-started from V ("Rotation, not just rescaling":
     L = U Lambda U^T): one step of simultaneous (subspace) iteration,
        P = L~ V,  P = Q R (Householder),  columns of Q flipped so that
        diag(R) >= 0,
     and Rayleigh quotients lam_i = max(q_i^T L~ q_i, 0).
  5. U <- Q re-quantized to 4 bits; lam stored as float32.

refresh_root()
  6. d_i = (lam_i + eps)^(-1/4)  ("Computing the inverse fourth root": damping
     before rooting), root codes <- current codes.

precondition(G)
  7. V^r = Bjorck^k(dequantize(root codes)) on each side and
        P_out = V^r_L diag(d_L) V^r_L^T  G  V^r_R diag(d_R) V^r_R^T
     i.e. L^(-1/4) G R^(-1/4) in the eigen form ("Where the fourth root comes
     from" for the exponent, "Rotation, not just rescaling" for the form).

Initial state: U = I (exact in the codebook), lam = 0, root = (I, d = 1), so
P_out = G until the first root refresh.

Diagonal fallback ("Blocked and distributed variants": if one dimension exceeds a
threshold, that side's factor is dropped and diagonal AdaGrad is used along it): a side
marked diagonal keeps no eigenvector matrix, only the diagonal of its factor as the same
exponential moving average,
    lam_i <- beta * lam_i + (1 - beta) * sum_j Gs[i, j]^2      (Gs: G for L, G^T for R)
and at a refresh d_i = (lam_i + eps)^(-1/4) like the eigenvalues of a full side; the
direction uses diag(d) in place of that side's root matrix.  Reading: the diagonal is
what diagonal AdaGrad accumulates along that dimension, and keeping the -1/4 exponent
keeps the step homogeneous of degree 0 and equal to the two-sided step whenever the
dropped factor is itself diagonal.

Parity status: steps 1-7 are pinned individually by the oracle tests
(codec round trips, Bjorck fixed points and convergence to the polar factor,
eigen refresh on exact eigenvectors and convergence to numpy.linalg.eigh,
closed-form roots, brute-force Kronecker preconditioner, homogeneity, the
diagonal / RMSprop special case).  The multi-step 4-bit trajectory as a whole
has no worked example on the pages: parity unpinned beyond those pins.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

from . import codec

SIDE_L = 0
SIDE_R = 1


# --------------------------------------------------------------------------
# Individual steps
# --------------------------------------------------------------------------

def bjorck(V, iters: int) -> np.ndarray:
    """Bjorck orthonormalization, ``iters`` times: V <- 1.5 V - 0.5 V (V^T V).

    Source: 4-bit Shampoo abstract ("rectifying the orthogonality of the
    quantized eigenvector matrix").
    """
    V = np.array(V, dtype=np.float64, copy=True)
    for _ in range(iters):
        V = 1.5 * V - 0.5 * (V @ (V.T @ V))
    return V


def rectified_eigenvectors(codes, scales, p: int, iters: int, qblock: int = 64,
                           codebook: str = codec.LINEAR_SQUARE) -> np.ndarray:
    """Steps 1-2: dequantize a side's eigenvector codes and rectify them."""
    Vt = codec.dequantize_matrix(codes, scales, p, qblock, codebook).astype(np.float64)
    return bjorck(Vt, iters)


def side_gradient(G, side: int) -> np.ndarray:
    """The gradient as seen by one side: G for L (G G^T), G^T for R (G^T G)."""
    G = np.asarray(G, dtype=np.float64)
    return G if side == SIDE_L else G.T


def statistics(V, lam, Gs, beta: float) -> np.ndarray:
    """Step 3: EMA statistic  beta * V diag(lam) V^T + (1 - beta) * Gs Gs^T.

    ``beta`` is used as the float32 value the device would hold.
    """
    b = np.float64(np.float32(beta))
    V = np.asarray(V, dtype=np.float64)
    lam = np.asarray(lam, dtype=np.float64)
    Gs = np.asarray(Gs, dtype=np.float64)
    return b * ((V * lam[None, :]) @ V.T) + (1.0 - b) * (Gs @ Gs.T)


def qr_positive(P) -> np.ndarray:
    """Householder QR (LAPACK) with columns of Q flipped so that diag(R) >= 0."""
    Q, R = np.linalg.qr(np.asarray(P, dtype=np.float64), mode="reduced")
    s = np.sign(np.diag(R))
    s[s == 0] = 1.0
    return Q * s[None, :]


def eigen_refresh(Lt, V, power_iters: int = 1):
    """Step 4: warm-started subspace iteration and Rayleigh quotients.

    Returns ``(Q, lam)`` in float64; ``lam`` is already clamped at zero.
    """
    Lt = np.asarray(Lt, dtype=np.float64)
    P = Lt @ np.asarray(V, dtype=np.float64)
    Q = None
    for it in range(max(1, power_iters)):
        Q = qr_positive(P)
        if it + 1 < power_iters:
            P = Lt @ Q
    lam = np.einsum("ij,ij->j", Q, Lt @ Q)
    return Q, np.maximum(lam, 0.0)


def root_scaling(lam32, eps: float) -> np.ndarray:
    """Step 6: d_i = (lam_i + eps)^(-1/4), from the stored float32 eigenvalues."""
    lam = np.asarray(lam32, dtype=np.float32).astype(np.float64)
    e = np.float64(np.float32(eps))
    return ((lam + e) ** -0.25).astype(np.float32)


def diagonal_statistics(lam, Gs, beta: float) -> np.ndarray:
    """Diagonal fallback statistic: beta * lam + (1 - beta) * (row sums of Gs^2), the
    diagonal of the EMA factor beta * L + (1 - beta) * Gs Gs^T (float64)."""
    b = np.float64(np.float32(beta))
    Gs = np.asarray(Gs, dtype=np.float64)
    return b * np.asarray(lam, dtype=np.float64) + (1.0 - b) * np.sum(Gs * Gs, axis=1)


def root_matrix(V, d) -> np.ndarray:
    """V diag(d) V^T (float64)."""
    V = np.asarray(V, dtype=np.float64)
    return (V * np.asarray(d, dtype=np.float64)[None, :]) @ V.T


def precondition_block(VL, dL, VR, dR, G) -> np.ndarray:
    """Step 7 (float64): V_L diag(d_L) V_L^T G V_R diag(d_R) V_R^T."""
    return root_matrix(VL, dL) @ np.asarray(G, dtype=np.float64) @ root_matrix(VR, dR)


# --------------------------------------------------------------------------
# State and the schedule
# --------------------------------------------------------------------------

@dataclass
class SideState:
    p: int
    codes: np.ndarray
    scales: np.ndarray
    lam: np.ndarray
    root_codes: np.ndarray
    root_scales: np.ndarray
    d: np.ndarray
    diagonal: bool = False      # diagonal fallback: no eigenvectors, lam is the diagonal
    # diagnostics of the last update (float64), for teacher-forced checks
    last_Lt: np.ndarray | None = field(default=None, repr=False)
    last_Q: np.ndarray | None = field(default=None, repr=False)

    def copy(self) -> "SideState":
        return SideState(self.p, self.codes.copy(), self.scales.copy(), self.lam.copy(),
                         self.root_codes.copy(), self.root_scales.copy(), self.d.copy(),
                         self.diagonal)


def initial_side(p: int, qblock: int = 64, codebook: str = codec.LINEAR_SQUARE,
                 diagonal: bool = False) -> SideState:
    if diagonal:
        empty_c, empty_s = np.zeros(0, np.uint8), np.zeros(0, np.float32)
        return SideState(p=p, codes=empty_c, scales=empty_s, lam=np.zeros(p, np.float32),
                         root_codes=empty_c.copy(), root_scales=empty_s.copy(),
                         d=np.ones(p, np.float32), diagonal=True)
    codes, scales = codec.quantize_matrix(np.eye(p, dtype=np.float32), qblock, codebook)
    return SideState(p=p, codes=codes, scales=scales,
                     lam=np.zeros(p, np.float32),
                     root_codes=codes.copy(), root_scales=scales.copy(),
                     d=np.ones(p, np.float32))


def update_side(st: SideState, Gs, beta: float, bjorck_iters: int,
                power_iters: int = 1, qblock: int = 64,
                codebook: str = codec.LINEAR_SQUARE) -> SideState:
    """Steps 1-5 for one side.  Returns the new state (root unchanged)."""
    if st.diagonal:
        out = st.copy()
        out.lam = diagonal_statistics(st.lam, Gs, beta).astype(np.float32)
        return out
    V = rectified_eigenvectors(st.codes, st.scales, st.p, bjorck_iters, qblock, codebook)
    Lt = statistics(V, st.lam, Gs, beta)
    Q, lam = eigen_refresh(Lt, V, power_iters)
    codes, scales = codec.quantize_matrix(Q.astype(np.float32), qblock, codebook)
    out = SideState(p=st.p, codes=codes, scales=scales, lam=lam.astype(np.float32),
                    root_codes=st.root_codes.copy(), root_scales=st.root_scales.copy(),
                    d=st.d.copy())
    out.last_Lt = Lt
    out.last_Q = Q
    return out


def refresh_side(st: SideState, eps: float) -> SideState:
    """Step 6 for one side."""
    out = st.copy()
    out.d = root_scaling(st.lam, eps)
    out.root_codes = st.codes.copy()
    out.root_scales = st.scales.copy()
    return out


def root_eigenvectors(st: SideState, bjorck_iters: int, qblock: int = 64,
                      codebook: str = codec.LINEAR_SQUARE) -> np.ndarray:
    """Rectified root eigenvectors (the identity for a diagonal side, whose root is diag(d))."""
    if st.diagonal:
        return np.eye(st.p)
    return rectified_eigenvectors(st.root_codes, st.root_scales, st.p, bjorck_iters, qblock, codebook)


class Shampoo4Oracle:
    """The whole schedule over a list of blocks (one SideState per block and side)."""

    def __init__(self, shapes, beta: float = 0.95, eps: float = 1e-6, qblock: int = 64,
                 bjorck_iters: int = 1, power_iters: int = 1, codebook: str = codec.LINEAR_SQUARE,
                 diagonal=None):
        """`diagonal`: per block a pair (side L diagonal, side R diagonal); default none."""
        self.shapes = [tuple(int(v) for v in s) for s in shapes]
        self.beta = beta
        self.eps = eps
        self.qblock = qblock
        self.bjorck_iters = bjorck_iters
        self.power_iters = power_iters
        self.codebook = codebook
        diagonal = diagonal or [(False, False)] * len(self.shapes)
        self.diagonal = [(bool(a), bool(b)) for a, b in diagonal]
        self.sides = [[initial_side(m, qblock, codebook, dl), initial_side(n, qblock, codebook, dr)]
                      for (m, n), (dl, dr) in zip(self.shapes, self.diagonal)]

    def update_stats(self, Gs):
        for b, G in enumerate(Gs):
            for side in (SIDE_L, SIDE_R):
                self.sides[b][side] = update_side(self.sides[b][side], side_gradient(G, side),
                                                  self.beta, self.bjorck_iters,
                                                  self.power_iters, self.qblock, self.codebook)

    def refresh_root(self):
        for b in range(len(self.shapes)):
            for side in (SIDE_L, SIDE_R):
                self.sides[b][side] = refresh_side(self.sides[b][side], self.eps)

    def precondition(self, Gs):
        out = []
        for b, G in enumerate(Gs):
            sl, sr = self.sides[b]
            X = np.asarray(G, dtype=np.float64)
            # L^(-1/4) G R^(-1/4); a diagonal side's root is diag(d)
            if sl.diagonal:
                X = sl.d.astype(np.float64)[:, None] * X
            else:
                X = root_matrix(root_eigenvectors(sl, self.bjorck_iters, self.qblock, self.codebook), sl.d) @ X
            if sr.diagonal:
                X = X * sr.d.astype(np.float64)[None, :]
            else:
                X = X @ root_matrix(root_eigenvectors(sr, self.bjorck_iters, self.qblock, self.codebook), sr.d)
            out.append(X.astype(np.float32))
        return out

    def step(self, Gs, t: int, root_interval: int = 1):
        """One block-step: update_stats, refresh_root when t % T == 0, precondition."""
        self.update_stats(Gs)
        if t % root_interval == 0:
            self.refresh_root()
        return self.precondition(Gs)
