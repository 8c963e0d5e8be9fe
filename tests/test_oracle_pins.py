"""Pins of the CPU oracle against what the pages and the mathematics fix.

Each test checks the oracle against something other than itself: a
hand-worked golden block, a closed form, an invariant, a library routine
(SciPy / NumPy LAPACK) or a brute-force full-matrix construction.  All CPU.
"""

from fractions import Fraction
import os

import numpy as np
import pytest
import scipy.linalg as sla

from oracle import bruteforce, codec
from oracle import shampoo4 as o

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rng(seed=0):
    return np.random.default_rng(seed)


def _random_orthogonal(p, rng):
    Q, R = np.linalg.qr(rng.standard_normal((p, p)))
    return Q * np.sign(np.diag(R))[None, :]


# ---------------------------------------------------------------------------
# Codec
# ---------------------------------------------------------------------------

def test_codebook_is_linear_square():
    """sqrt|q_j| (signed) is the uniform grid -1 + 2j/15, except the exact zero at j = 7."""
    lv = codec.exact_levels()
    assert lv[7] == 0
    for j in range(16):
        if j == 7:
            continue
        q = lv[j]
        t = Fraction(-1) + Fraction(2 * j, 15)
        # signed square root of q equals t exactly  <=>  q == sign(t) t^2 with |t| rational
        assert abs(q) == t * t
        assert (q > 0) == (t > 0)
    # float32 table is the correctly rounded exact table (half-ulp bound)
    for j, q in enumerate(lv):
        f = codec.LEVELS[j]
        if q == 0:
            assert f == 0
            continue
        ulp = np.spacing(np.float32(abs(f)))
        assert abs(Fraction(float(f)) - q) <= Fraction(float(ulp)) / 2
    assert np.all(np.diff(codec.LEVELS) > 0)
    assert np.all(np.diff(codec.MIDPOINTS) > 0)
    assert codec.LEVELS[0] == -1.0 and codec.LEVELS[15] == 1.0


def _load_golden_block():
    vals, codes, packed, scale = [], [], None, None
    for line in open(os.path.join(GOLDEN, "codec_block.txt")):
        line = line.strip()
        if not line or line.startswith("#"):
            continue
        if line.startswith("packed"):
            packed = bytes(int(h, 16) for h in line.split()[1:])
        elif line.startswith("scale"):
            scale = float(line.split()[1])
        else:
            v, c = line.split()
            vals.append(float(v))
            codes.append(int(c))
    return vals, codes, packed, scale


def test_golden_hand_worked_block():
    vals, codes, packed, scale = _load_golden_block()
    x = np.zeros(64, np.float32)
    x[: len(vals)] = vals
    got_codes, got_scales = codec.quantize(x, 64)
    assert got_scales.tolist() == [np.float32(scale)]
    assert bytes(got_codes.tolist()) == packed
    unpacked = codec.unpack_nibbles(got_codes)
    assert unpacked[: len(codes)].tolist() == codes


def _codes_for_xhat(xhat):
    """Codes for normalized values, using blocks whose absmax is exactly 1."""
    xhat = np.asarray(xhat, np.float32)
    n = xhat.size
    per = 63
    nb = (n + per - 1) // per
    blocks = np.zeros((nb, 64), np.float32)
    blocks[:, 0] = 1.0
    flat = np.zeros(nb * per, np.float32)
    flat[:n] = xhat
    blocks[:, 1:] = flat.reshape(nb, per)
    c, s = codec.quantize(blocks.ravel(), 64)
    assert np.all(s == 1.0)
    return codec.unpack_nibbles(c).reshape(nb, 64)[:, 1:].ravel()[:n]


def _exact_nearest(xf: float):
    """Nearest exact level by exact rational distance; ties -> lower code."""
    x = Fraction(xf)
    best, bestd = None, None
    for j, q in enumerate(codec.exact_levels()):
        d = abs(x - q)
        if bestd is None or d < bestd:
            best, bestd = j, d
    return best


def test_quantize_matches_bruteforce_nearest_level():
    """Codes equal the exact nearest level, except only inside the float32 rounding
    interval of a midpoint (where the float32 midpoint decides)."""
    rng = _rng(1)
    samples = [rng.uniform(-1, 1, 4000).astype(np.float32)]
    # dense neighbourhoods of every midpoint (+-40 ulps)
    for m in codec.MIDPOINTS:
        around = [m]
        up = down = np.float32(m)
        for _ in range(40):
            up = np.nextafter(up, np.float32(2))
            down = np.nextafter(down, np.float32(-2))
            around += [up, down]
        samples.append(np.array(around, np.float32))
    samples.append(np.array([0.0, -0.0, 1.0, -1.0, 1e-40, -1e-40, 1e-30], np.float32))
    xs = np.concatenate(samples)
    got = _codes_for_xhat(xs)
    exact_mids = codec.exact_midpoints()
    for x, c in zip(xs.tolist(), got.tolist()):
        e = _exact_nearest(x)
        if c == e:
            continue
        # disagreement allowed only between an exact midpoint and its float32 rounding
        j = min(c, e)
        assert abs(c - e) == 1
        fm = Fraction(float(codec.MIDPOINTS[j]))
        lo, hi = sorted([fm, exact_mids[j]])
        assert lo <= Fraction(x) <= hi, (x, c, e)


def test_ties_go_to_lower_code():
    got = _codes_for_xhat(codec.MIDPOINTS)
    assert got.tolist() == list(range(15))
    nxt = np.nextafter(codec.MIDPOINTS, np.float32(2))
    assert _codes_for_xhat(nxt).tolist() == list(range(1, 16))


def test_round_trip_exact_on_codebook_values():
    rng = _rng(2)
    for trial in range(50):
        s = np.float32(10.0 ** rng.uniform(-6, 3))
        codes = rng.integers(0, 16, 64)
        codes[rng.integers(0, 64)] = rng.choice([0, 15])   # absmax level present
        x = (codec.LEVELS[codes] * s).astype(np.float32)
        c, sc = codec.quantize(x, 64)
        assert sc[0] == s
        assert codec.unpack_nibbles(c).tolist() == codes.tolist()
        y = codec.dequantize(c, sc, 64, 64)
        assert np.array_equal(y.view(np.uint32), x.view(np.uint32))


@pytest.mark.parametrize("p", [1, 2, 3, 7, 31, 32, 33, 64, 65, 100, 256, 1024])
def test_identity_is_exact(p):
    c, s = codec.quantize_matrix(np.eye(p, dtype=np.float32))
    V = codec.dequantize_matrix(c, s, p)
    assert np.array_equal(V, np.eye(p, dtype=np.float32))
    assert c.size == codec.num_qblocks(p * p) * 32


def test_zero_and_padding_blocks():
    x = np.zeros(130, np.float32)
    x[70] = -3.0
    c, s = codec.quantize(x, 64)
    assert s.tolist() == [0.0, 3.0, 0.0]
    u = codec.unpack_nibbles(c)
    assert u.size == 192
    assert np.all(u[:64] == 7) and np.all(u[130:] == 7)
    assert u[70] == 0
    y = codec.dequantize(c, s, 130)
    assert np.array_equal(y, x)
    # signed zero and subnormal blocks
    z = np.array([-0.0, 0.0] * 32, np.float32)
    cz, sz = codec.quantize(z)
    assert sz[0] == 0 and np.all(codec.unpack_nibbles(cz) == 7)
    sub = np.zeros(64, np.float32)
    sub[0] = np.float32(3e-42)
    sub[5] = -np.float32(3e-42)
    cs, ss = codec.quantize(sub)
    assert ss[0] == np.float32(3e-42)
    assert np.array_equal(codec.dequantize(cs, ss, 64), sub)


def test_nibble_order():
    codes = np.arange(16, dtype=np.uint8)
    packed = codec.pack_nibbles(codes)
    assert packed.tolist() == [0x10, 0x32, 0x54, 0x76, 0x98, 0xBA, 0xDC, 0xFE]
    assert codec.unpack_nibbles(packed).tolist() == codes.tolist()


# ---------------------------------------------------------------------------
# Bjorck
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("p", [1, 5, 32])
def test_bjorck_fixes_signed_permutations_bitwise(p):
    rng = _rng(3)
    P = np.eye(p)[rng.permutation(p)] * rng.choice([-1.0, 1.0], p)[:, None]
    for k in (1, 3):
        assert np.array_equal(o.bjorck(P, k), P)


def test_bjorck_converges_to_polar_factor():
    rng = _rng(4)
    p = 24
    U = _random_orthogonal(p, rng)
    Vt = U + 0.05 * rng.standard_normal((p, p))
    assert np.linalg.norm(Vt.T @ Vt - np.eye(p), 2) < 1
    polar_u, _ = sla.polar(Vt)
    V = o.bjorck(Vt, 30)
    assert np.max(np.abs(V - polar_u)) < 1e-12
    # quadratic convergence: one step squares the orthogonality defect (to first order)
    e0 = np.linalg.norm(Vt.T @ Vt - np.eye(p), 2)
    V1 = o.bjorck(Vt, 1)
    e1 = np.linalg.norm(V1.T @ V1 - np.eye(p), 2)
    assert e1 < 1.5 * e0 ** 2


def test_bjorck_on_quantized_orthogonal_matrix_reduces_defect():
    rng = _rng(5)
    p = 64
    U = _random_orthogonal(p, rng).astype(np.float32)
    c, s = codec.quantize_matrix(U)
    Vt = codec.dequantize_matrix(c, s, p).astype(np.float64)
    e0 = np.linalg.norm(Vt.T @ Vt - np.eye(p))
    V = o.bjorck(Vt, 1)
    e1 = np.linalg.norm(V.T @ V - np.eye(p))
    assert e1 < 0.5 * e0
    # the polar factor is closer to U than the raw dequantized matrix
    polar_u, _ = sla.polar(Vt)
    assert np.linalg.norm(polar_u - U) < np.linalg.norm(Vt - U)


# ---------------------------------------------------------------------------
# Statistics
# ---------------------------------------------------------------------------

def test_statistics_sum_of_outer_products_and_equivariance():
    rng = _rng(6)
    p, q = 6, 4
    V = _random_orthogonal(p, rng)
    lam = rng.uniform(0, 2, p)
    G = rng.standard_normal((p, q))
    beta = 0.9
    Lt = o.statistics(V, lam, G, beta)
    b = np.float64(np.float32(beta))
    ref = np.zeros((p, p))
    for i in range(p):
        ref += b * lam[i] * np.outer(V[:, i], V[:, i])
    for c in range(q):
        ref += (1 - b) * np.outer(G[:, c], G[:, c])
    assert np.allclose(Lt, ref, rtol=1e-13, atol=1e-13)
    assert np.allclose(Lt, Lt.T)
    assert np.min(np.linalg.eigvalsh(Lt)) > -1e-12
    # rotating the row space rotates the statistic
    U = _random_orthogonal(p, rng)
    Lr = o.statistics(U @ V, lam, U @ G, beta)
    assert np.allclose(Lr, U @ Lt @ U.T, atol=1e-12)


def test_side_gradient_orientation():
    G = np.arange(6.0).reshape(2, 3)
    assert o.statistics(np.eye(2), np.zeros(2), o.side_gradient(G, o.SIDE_L), 0.0).shape == (2, 2)
    assert o.statistics(np.eye(3), np.zeros(3), o.side_gradient(G, o.SIDE_R), 0.0).shape == (3, 3)


# ---------------------------------------------------------------------------
# Eigen refresh
# ---------------------------------------------------------------------------

def test_refresh_on_exact_eigenvectors_is_exact():
    rng = _rng(7)
    p = 16
    U = _random_orthogonal(p, rng)
    mu = rng.uniform(0.5, 5.0, p)
    L = (U * mu) @ U.T
    Q, lam = o.eigen_refresh(L, U)
    assert np.max(np.abs(Q - U)) < 1e-12          # signs kept: R_jj = mu_j > 0
    assert np.max(np.abs(lam - mu)) < 1e-12
    # flipped warm start still returns the same signs as the warm start
    Uf = U * rng.choice([-1.0, 1.0], p)[None, :]
    Qf, _ = o.eigen_refresh(L, Uf)
    assert np.max(np.abs(Qf - Uf)) < 1e-12


def test_refresh_diagonal_with_identity_warm_start():
    d = np.array([3.0, 0.0, 1.0, 7.0, 0.5])
    Q, lam = o.eigen_refresh(np.diag(d), np.eye(5))
    assert np.array_equal(Q, np.eye(5))
    assert np.array_equal(lam, d)


def test_qr_positive_diagonal():
    rng = _rng(8)
    P = rng.standard_normal((12, 12))
    Q = o.qr_positive(P)
    R = Q.T @ P
    assert np.allclose(np.tril(R, -1), 0, atol=1e-12)
    assert np.all(np.diag(R) >= 0)
    assert np.allclose(Q.T @ Q, np.eye(12), atol=1e-13)


def test_repeated_refresh_converges_to_eigh():
    rng = _rng(9)
    p = 10
    U = _random_orthogonal(p, rng)
    mu = 2.0 ** -np.arange(p)           # well separated
    L = (U * mu) @ U.T
    V = np.eye(p)
    for _ in range(200):
        V, lam = o.eigen_refresh(L, V)
    w, W = np.linalg.eigh(L)
    order = np.argsort(w)[::-1]
    assert np.allclose(lam, w[order], rtol=1e-10, atol=1e-14)
    # same eigenvectors up to sign
    assert np.allclose(np.abs(np.sum(V * W[:, order], axis=0)), 1.0, atol=1e-8)


# ---------------------------------------------------------------------------
# Root
# ---------------------------------------------------------------------------

def test_root_diagonal_closed_form():
    lam = np.array([0.0, 1e-6, 1.0, 16.0, 81.0], np.float32)
    eps = 1e-6
    d = o.root_scaling(lam, eps)
    e = float(np.float32(eps))
    expect = np.array([(float(v) + e) ** -0.25 for v in lam], np.float32)
    assert np.allclose(d, expect, rtol=1e-7)
    assert d[3] == np.float32((16.0 + e) ** -0.25)
    assert abs(float(o.root_scaling(np.array([16.0], np.float32), 0.0)[0]) - 0.5) == 0
    assert abs(float(o.root_scaling(np.array([81.0], np.float32), 0.0)[0]) - 1 / 3) < 1e-7


def test_root_fourth_power_inverts():
    rng = _rng(10)
    p = 12
    A = rng.standard_normal((p, p))
    L = A @ A.T + 0.1 * np.eye(p)
    w, U = np.linalg.eigh(L)
    Rt = o.root_matrix(U, w ** -0.25)
    assert np.allclose(np.linalg.matrix_power(Rt, 4) @ L, np.eye(p), atol=1e-9)


# ---------------------------------------------------------------------------
# Precondition vs brute-force Kronecker construction
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("m,n", [(2, 3), (4, 4), (6, 5), (3, 6)])
def test_precondition_matches_kronecker_bruteforce(m, n):
    rng = _rng(11 + m * 7 + n)
    Gs = [rng.standard_normal((m, n)) for _ in range(4)]
    L = sum(G @ G.T for G in Gs) + 0.01 * np.eye(m)
    R = sum(G.T @ G for G in Gs) + 0.01 * np.eye(n)
    wl, UL = np.linalg.eigh(L)
    wr, UR = np.linalg.eigh(R)
    got = o.precondition_block(UL, wl ** -0.25, UR, wr ** -0.25, Gs[-1])
    ref = bruteforce.kronecker_root_direction(L, R, Gs[-1])
    assert np.allclose(got, ref, rtol=1e-9, atol=1e-11)


def test_vec_identity_convention():
    rng = _rng(12)
    A = rng.standard_normal((3, 3))
    B = rng.standard_normal((2, 2))
    X = rng.standard_normal((2, 3))
    lhs = np.kron(A, B) @ bruteforce.vec(X)
    assert np.allclose(lhs, bruteforce.vec(B @ X @ A.T))


def test_kronecker_bound_needs_rank_factor():
    """The dominance H <= R^(1/2) kron L^(1/2) holds with the rank factor r;
    as printed (no factor) it fails already for G = I_2."""
    G = np.eye(2)
    H = bruteforce.full_adagrad_statistic([G])
    K = np.kron(bruteforce.psd_sqrt(G.T @ G), bruteforce.psd_sqrt(G @ G.T))
    assert np.min(np.linalg.eigvalsh(K - H)) < -0.5
    assert np.min(np.linalg.eigvalsh(2 * K - H)) > -1e-12
    rng = _rng(13)
    for trial in range(20):
        m, n = rng.integers(2, 5, 2)
        Gs = [rng.standard_normal((m, n)) for _ in range(rng.integers(1, 4))]
        r = max(np.linalg.matrix_rank(G) for G in Gs)
        H = bruteforce.full_adagrad_statistic(Gs)
        L = sum(G @ G.T for G in Gs)
        R = sum(G.T @ G for G in Gs)
        K = np.kron(bruteforce.psd_sqrt(R), bruteforce.psd_sqrt(L))
        assert np.min(np.linalg.eigvalsh(r * K - H)) > -1e-9


# ---------------------------------------------------------------------------
# Whole schedule: homogeneity and the diagonal (RMSprop) special case
# ---------------------------------------------------------------------------

def test_degree_zero_homogeneity():
    rng = _rng(14)
    m, n = 7, 7          # square and full rank, so eps = 0 is well defined from step 1
    Gs = [rng.standard_normal((m, n)).astype(np.float32) for _ in range(4)]
    a = o.Shampoo4Oracle([(m, n)], beta=0.9, eps=0.0)
    b = o.Shampoo4Oracle([(m, n)], beta=0.9, eps=0.0)
    for t, G in enumerate(Gs, start=1):
        Pa = a.step([G], t)[0]
        Pb = b.step([np.float32(2) * G], t)[0]
        for s in (0, 1):
            assert np.array_equal(a.sides[0][s].codes, b.sides[0][s].codes)
        # equal up to the float32 rounding of d = (lam + eps)^(-1/4) and of P_out
        assert np.linalg.norm(Pa - Pb) <= 1e-6 * np.linalg.norm(Pa)
    # with the default eps the step is only approximately homogeneous
    c = o.Shampoo4Oracle([(m, n)], beta=0.9, eps=1e-6)
    d = o.Shampoo4Oracle([(m, n)], beta=0.9, eps=1e-6)
    for t, G in enumerate(Gs, start=1):
        Pc = c.step([G], t)[0]
        Pd = d.step([np.float32(2) * G], t)[0]
    assert np.allclose(Pc, Pd, rtol=1e-3)


def test_diagonal_gradients_reduce_to_rmsprop():
    """Square diagonal gradients keep U = I, so the step is RMSprop (no momentum)
    with eps inside the square root: v <- beta v + (1 - beta) g^2,
    update = g / sqrt(v + eps)."""
    rng = _rng(15)
    p = 16
    beta, eps = 0.95, 1e-6
    orc = o.Shampoo4Oracle([(p, p)], beta=beta, eps=eps)
    v = np.zeros(p, np.float32)
    b32 = np.float32(beta)
    for t in range(1, 8):
        g = rng.standard_normal(p).astype(np.float32) * np.float32(10.0) ** rng.uniform(-1, 1, p).astype(np.float32)
        if t == 3:
            g[:3] = 0
        G = np.diag(g)
        P = orc.step([G], t)[0]
        # textbook RMSprop accumulator, float64 math rounded to float32 like the stored eigenvalues
        v = (np.float64(b32) * v + (1.0 - np.float64(b32)) * g.astype(np.float64) ** 2).astype(np.float32)
        upd = g / np.sqrt(v.astype(np.float64) + float(np.float32(eps)))
        assert np.allclose(np.diag(P), upd, rtol=1e-6, atol=1e-30)
        assert np.count_nonzero(P - np.diag(np.diag(P))) == 0
        for s in (0, 1):
            st = orc.sides[0][s]
            assert np.array_equal(codec.dequantize_matrix(st.codes, st.scales, p), np.eye(p, dtype=np.float32))


def test_initial_root_is_identity():
    rng = _rng(16)
    orc = o.Shampoo4Oracle([(5, 3)])
    G = rng.standard_normal((5, 3)).astype(np.float32)
    assert np.array_equal(orc.precondition([G])[0], G)


# ---------------------------------------------------------------------------
# Root refresh every T > 1 steps ("The cost dial": accumulate every step,
# recompute the roots only every T steps)
# ---------------------------------------------------------------------------

def test_diagonal_gradients_with_stale_root_between_refreshes():
    """Square diagonal gradients with the root refreshed every T = 3 steps: the
    eigenvalues follow the RMSprop accumulator at every step, but the direction uses
    the accumulator as it was at the last refresh, g_t / sqrt(v_tau + eps) with
    tau = 3 * floor(t / 3), and the identity root (P = G) before the first refresh.
    A schedule that refreshed every step, or that paired the current eigenvalues with
    the stale root, fails."""
    rng = _rng(17)
    p, T = 12, 3
    beta, eps = 0.9, 1e-6
    orc = o.Shampoo4Oracle([(p, p)], beta=beta, eps=eps)
    v = np.zeros(p, np.float32)
    v_root = None
    b32 = np.float32(beta)
    for t in range(1, 11):
        g = rng.standard_normal(p).astype(np.float32) * np.float32(10.0) ** rng.uniform(-1, 1, p).astype(np.float32)
        P = orc.step([np.diag(g)], t, root_interval=T)[0]
        v = (np.float64(b32) * v + (1.0 - np.float64(b32)) * g.astype(np.float64) ** 2).astype(np.float32)
        for s in (0, 1):
            assert np.allclose(orc.sides[0][s].lam, v, rtol=1e-6, atol=1e-30)
        if t % T == 0:
            v_root = v.copy()
        if v_root is None:
            assert np.array_equal(P, np.diag(g))
        else:
            upd = g / np.sqrt(v_root.astype(np.float64) + float(np.float32(eps)))
            assert np.allclose(np.diag(P), upd, rtol=1e-6, atol=1e-30), t
            if t % T != 0:
                # the current accumulator differs from the one the root was taken from
                assert not np.allclose(np.diag(P), g / np.sqrt(v.astype(np.float64) + eps), rtol=1e-4)
        assert np.count_nonzero(P - np.diag(np.diag(P))) == 0


def test_root_snapshot_is_the_state_at_the_last_refresh():
    """Between refreshes the root codes and d stay those taken at the last refresh while
    the statistics state moves on every step (general, non-diagonal gradients)."""
    rng = _rng(18)
    m, n, T = 9, 6, 4
    orc = o.Shampoo4Oracle([(m, n)], beta=0.9, eps=1e-6)
    snap = None
    for t in range(1, 10):
        G = rng.standard_normal((m, n)).astype(np.float32)
        orc.step([G], t, root_interval=T)
        sides = orc.sides[0]
        if t % T == 0:
            snap = [(s.codes.copy(), s.scales.copy(), o.root_scaling(s.lam, 1e-6)) for s in sides]
        for s_, st in enumerate(sides):
            if snap is None:
                ref = o.initial_side(st.p)
                assert np.array_equal(st.root_codes, ref.codes) and np.all(st.d == 1)
            else:
                c, sc, d = snap[s_]
                assert np.array_equal(st.root_codes, c) and np.array_equal(st.root_scales, sc)
                assert np.array_equal(st.d, d)


def test_degree_zero_homogeneity_with_root_interval():
    """Homogeneity holds for the whole schedule at T = 3 too: codes bit-identical under
    G -> 2G and directions equal at eps = 0 (from step 1 the identity root gives P = G,
    which scales; from the first refresh on the step is invariant)."""
    rng = _rng(19)
    m, n, T = 6, 6, 3
    Gs = [rng.standard_normal((m, n)).astype(np.float32) for _ in range(7)]
    a = o.Shampoo4Oracle([(m, n)], beta=0.9, eps=0.0)
    b = o.Shampoo4Oracle([(m, n)], beta=0.9, eps=0.0)
    for t, G in enumerate(Gs, start=1):
        Pa = a.step([G], t, root_interval=T)[0]
        Pb = b.step([np.float32(2) * G], t, root_interval=T)[0]
        for s in (0, 1):
            assert np.array_equal(a.sides[0][s].codes, b.sides[0][s].codes)
            assert np.array_equal(a.sides[0][s].root_codes, b.sides[0][s].root_codes)
        if t < T:
            assert np.array_equal(Pb, np.float32(2) * Pa)
        else:
            assert np.linalg.norm(Pa - Pb) <= 1e-6 * np.linalg.norm(Pa), t
