"""Teacher-forced parity of the whole step against the CPU oracle.

Every step starts the oracle from the state the GPU held before the step (codes,
scales, eigenvalues, root snapshot), and the oracle computes the whole step from it:
  update_stats   the rectified eigenvectors from the GPU's codes, the statistic from
                 them, the GPU's eigenvalues and G, the refresh from that statistic;
                 compared are the statistic, the basis-invariant product
                 Q diag(lam) Q^T and the eigenvalues (rel-Frobenius <= 1e-3), and the
                 new codes, which must equal the oracle codec applied to the GPU's own
                 fp32 Q bit for bit (the codec in isolation);
  refresh_root   d and the root codes, and with cached roots the root matrices
                 V^r diag(d) V^r^T;
  precondition   the preconditioned gradient, with the root the oracle itself takes at
                 a refresh step (its own codes of its own Q, its own d) and the GPU's
                 pre-step root otherwise (rel-Frobenius <= 1e-3); and again from the
                 root the GPU holds after the step.
Eigenvalues below the float32 floor (about p u lam_max, see `resolved`) are not fixed
by the float32 path: there d is compared where resolved (element by element, within
the bound the floor implies), the GPU's eigenvalue is checked to lie in the range
float32 allows, and the preconditioned gradient and root matrices of that refresh are
compared from the GPU's own root (the gap to the oracle's own root is reported).  When
every eigenvalue is resolved, the oracle's own root is used with the GPU's d only for
the eigenvalues within 250x the floor (those d are correct values within their bound).
`use_step` runs the step as one shampoo4_step call (the benchmark's path: with cached
roots and no refresh due the precondition runs beside the statistics update);
otherwise as the three calls.
Where several results are correct (the basis of an eigenspace of a repeated or
zero eigenvalue), only basis-invariant products are compared.
"""

import numpy as np
import pytest
import torch

from oracle import codec
from oracle import shampoo4 as o
from tests.gpu_util import announce, rel_fro, require_gpu, to_dev
from workloads import get_workload

pytestmark = pytest.mark.gpu

TOL = 1e-3
BUF_ROOT_MAT = 20
U32 = 2.0 ** -24     # float32 unit roundoff
U64 = 2.0 ** -53     # float64 unit roundoff


def resolved(lam, p, u=U32, P=None, Q=None):
    """Eigenvalues float32 arithmetic determines: a Rayleigh quotient of an order-p
    statistic computed in float32 (and the statistic itself) carries an absolute error
    of up to about p u |L|, so eigenvalues below p u lam_max are not fixed by the
    float32 path: any value in [0, ~2 p u lam_max] is a correct result there, and
    d = (lam + eps)^(-1/4) with it.
    The refresh takes its eigenvectors from the QR of P = L V (one warm-started power
    step, not a converged eigensolver).  Householder QR is backward stable column by
    column, so column j of Q is fixed only to about u / min_{i <= j} sin(angle between p_i
    and p_1 .. p_{i-1}); where P's columns are close to dependent (a rank-deficient
    statistic whose warm start spans more than its range), the Rayleigh quotient of column
    j moves by that factor more.  With P (the last QR's input) and Q (its orthonormal
    factor) given, column j's floor is p u lam_max / min_{i <= j} (|R_ii| / |p_i|), R = Q^T P.
    Returns (mask of resolved eigenvalues, per-eigenvalue threshold)."""
    lam = np.asarray(lam, np.float64)
    thr = p * u * float(lam.max()) if lam.size else 0.0
    thr = np.full(lam.shape, thr)
    if P is not None and lam.size:
        rd = np.abs(np.einsum("ij,ij->j", Q, P))
        sines = rd / np.maximum(np.linalg.norm(P, axis=0), 1e-300)
        thr = thr / np.maximum(np.minimum.accumulate(sines), 1e-300)
    return lam > thr, thr


def _run_teacher_forced(shapes, grads_fn, steps, beta=0.95, eps=1e-6, k=1, power_iters=1,
                        root_interval=1, root_cache=False, label="", qr="auto", codebook="ls",
                        sample=None, all_sides=None, use_step=False, check_from=1, fp64=False):
    """`sample`: the blocks checked against the oracle (default: every block).
    `all_sides(blocks, t)`: an optional extra check after each statistics update.
    `check_from`: the first step checked; earlier steps run on the GPU only (a long
    schedule is checked in windows, one test each)."""
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    cfg = Shampoo4Config(beta=beta, eps=eps, bjorck_iters=k, power_iters=power_iters,
                         root_cache=root_cache, qr_schedule=qr, codebook=codebook, fp64_refresh=fp64)
    unit = U64 if fp64 else U32
    announce(f"step parity {label}: init {len(shapes)} blocks")
    blocks = Shampoo4Blocks(shapes, cfg)
    torch.cuda.synchronize()
    checked = list(range(len(shapes))) if sample is None else list(sample)
    # initial state equals the oracle's
    for b in checked:
        m, n = shapes[b]
        for s, p in ((0, m), (1, n)):
            ref = o.initial_side(p, 64, codebook)
            got = blocks.side_state(b, s)
            assert np.array_equal(got["codes"], ref.codes)
            assert np.array_equal(got["scales"], ref.scales)
            assert np.array_equal(got["root_codes"], ref.root_codes)
            assert np.all(got["lam"] == 0) and np.all(got["d"] == 1)
            if root_cache:
                assert np.array_equal(blocks.view(b, s, BUF_ROOT_MAT).cpu().numpy(), np.eye(p, dtype=np.float32))
    worst = {"stat": 0.0, "recon": 0.0, "lam": 0.0, "P": 0.0, "P_gpu_root": 0.0, "root_mat": 0.0, "d": 0.0,
             "P_unresolved": 0.0}
    n_unresolved = 0     # refresh steps of checked blocks with eigenvalues below the float32 floor
    flips = [0, 0]      # codes that differ from the oracle's own codes of its own Q, and codes compared
    for t in range(1, steps + 1):
        Gs = grads_fn(t)
        Gd = [to_dev(G) for G in Gs]
        refresh = t % root_interval == 0
        if t < check_from:
            if t == 1 or t % 10 == 0:
                announce(f"step parity {label}: t={t} (GPU only)")
            blocks.step(Gd, t, root_interval)
            continue
        before = {b: [blocks.side_state(b, s) for s in (0, 1)] for b in checked}
        if use_step:
            announce(f"step parity {label}: t={t} step (refresh={refresh})")
            outs = blocks.step(Gd, t, root_interval)
        else:
            announce(f"step parity {label}: t={t} update_stats")
            blocks.update_stats(Gd)
        torch.cuda.synchronize()
        if all_sides is not None:
            all_sides(blocks, t)
        new_root = {}   # the oracle's own root at a refresh step, from the pre-step state
        for b in checked:
            m, n = shapes[b]
            for s, p in ((0, m), (1, n)):
                st = before[b][s]
                Gs_side = o.side_gradient(Gs[b], s)
                V = o.rectified_eigenvectors(st["codes"], st["scales"], p, k, 64, codebook)
                Lt_ref = o.statistics(V, st["lam"], Gs_side, beta)
                Lt_gpu = blocks.view(b, s, 21 if fp64 else 17).cpu().numpy().astype(np.float64)
                # symmetric up to the float32 rounding of the K-scaled products (off-diagonal
                # tiles are stored mirrored)
                assert rel_fro(Lt_gpu, Lt_gpu.T) <= 1e-6, (label, t, b, s, "statistic not symmetric")
                e_stat = rel_fro(Lt_gpu, Lt_ref)
                assert e_stat <= TOL, (label, t, b, s, "statistic", e_stat)
                Q_ref, lam_ref = o.eigen_refresh(Lt_ref, V, power_iters)
                Q_gpu32 = blocks.view(b, s, 18).cpu().numpy()
                after = blocks.side_state(b, s)
                lam_gpu = after["lam"].astype(np.float64)
                Q_gpu = blocks.view(b, s, 22).cpu().numpy() if fp64 else Q_gpu32.astype(np.float64)
                e_rec = rel_fro((Q_gpu * lam_gpu) @ Q_gpu.T, (Q_ref * lam_ref) @ Q_ref.T)
                e_lam = rel_fro(lam_gpu, lam_ref)
                assert e_rec <= TOL, (label, t, b, s, "Q diag(lam) Q^T", e_rec)
                assert e_lam <= TOL, (label, t, b, s, "eigenvalues", e_lam)
                assert np.allclose(Q_gpu.T @ Q_gpu, np.eye(p), atol=1e-4), (label, t, b, s, "orthonormal Q")
                c_ref, s_ref = codec.quantize_matrix(Q_gpu32, 64, codebook)
                assert np.array_equal(after["codes"], c_ref), (label, t, b, s, "codes")
                assert np.array_equal(after["scales"].view(np.uint32), s_ref.view(np.uint32))
                c_own, s_own = codec.quantize_matrix(Q_ref.astype(np.float32), 64, codebook)
                lo = lambda c: np.stack([c & 15, c >> 4], -1)
                flips[0] += int(np.count_nonzero(lo(c_own) != lo(after["codes"])))
                flips[1] += 2 * c_own.size
                if refresh:
                    d_own = o.root_scaling(lam_ref.astype(np.float32), eps)
                    P_last = Lt_ref @ V
                    for _ in range(power_iters - 1):
                        P_last = Lt_ref @ o.qr_positive(P_last)
                    mask, thr = resolved(lam_ref, p, unit, P_last, Q_ref)
                    same = bool(np.array_equal(c_own, after["codes"]) and
                                np.array_equal(s_own.view(np.uint32), after["scales"].view(np.uint32)))
                    new_root[(b, s)] = (c_own, s_own, d_own, mask, thr, same)
                worst["stat"] = max(worst["stat"], e_stat)
                worst["recon"] = max(worst["recon"], e_rec)
                worst["lam"] = max(worst["lam"], e_lam)
        if refresh:
            if not use_step:
                announce(f"step parity {label}: t={t} refresh_root")
                blocks.refresh_root()
                torch.cuda.synchronize()
            for b in checked:
                for s in (0, 1):
                    st = blocks.side_state(b, s)
                    assert np.array_equal(st["root_codes"], st["codes"])
                    assert np.array_equal(st["root_scales"], st["scales"])
                    d_ref = o.root_scaling(st["lam"], eps)
                    assert np.allclose(st["d"], d_ref, rtol=2e-6, atol=0), (label, t, b, s, "d")
                    _, _, d_own, mask, thr, _ = new_root[(b, s)]
                    lam_own = d_own.astype(np.float64) ** -4 - eps
                    # d from the pre-step state where float32 resolves the eigenvalue, element
                    # by element within 1e-3 plus what an eigenvalue error of up to 2 p u lam_max
                    # moves (lam + eps)^(-1/4) by; below the floor the GPU's eigenvalue must lie
                    # in the range float32 allows
                    rel = np.abs(st["d"].astype(np.float64) / d_own - 1.0)
                    bound = TOL + 0.5 * thr / (np.maximum(lam_own, 0.0) + eps)
                    assert np.all(rel[mask] <= bound[mask]), (label, t, b, s, "d from the pre-step state",
                                                              float((rel - bound)[mask].max()))
                    assert np.all(st["lam"][~mask] <= lam_own[~mask] + 2 * thr[~mask]), \
                        (label, t, b, s, "unresolved eigenvalue range")
                    worst["d"] = max(worst["d"], float(rel[mask].max()) if mask.any() else 0.0)
        if not use_step:
            announce(f"step parity {label}: t={t} precondition")
            outs = blocks.precondition(Gd)
            torch.cuda.synchronize()
        for P in outs:
            assert bool(torch.isfinite(P).all()), (label, t, "non-finite preconditioned gradient")
        for b in checked:
            m, n = shapes[b]
            P_gpu = outs[b].cpu().numpy()
            # (1) the whole step from the pre-step state: at a refresh the oracle's own root
            roots = []
            all_resolved = True
            for s, p in ((0, m), (1, n)):
                if refresh:
                    c, sc, d, mask, thr, same = new_root[(b, s)]
                    all_resolved = all_resolved and bool(mask.all()) and same
                    # where an eigenvalue is within 250x the float32 floor its d is known only
                    # to within the bound checked above: take the GPU's (a correct value), the
                    # oracle's everywhere else
                    lam_own = d.astype(np.float64) ** -4 - eps
                    d = np.where(lam_own + eps >= 250 * thr, d, blocks.side_state(b, s)["d"]).astype(np.float32)
                else:
                    st = before[b][s]
                    c, sc, d = st["root_codes"], st["root_scales"], st["d"]
                roots.append((o.rectified_eigenvectors(c, sc, p, k, 64, codebook), d))
            P_ref = o.precondition_block(roots[0][0], roots[0][1], roots[1][0], roots[1][1], Gs[b])
            e_p = rel_fro(P_gpu, P_ref)
            if all_resolved:
                assert e_p <= TOL, (label, t, b, "P from the pre-step state", e_p)
                worst["P"] = max(worst["P"], e_p)
            else:
                # unresolved eigenvalues, or the oracle's codes of its own Q differ from the
                # GPU's (eigenvectors of a cluster or null space are fixed only up to a
                # rotation, which the 4-bit encoding turns into other codes): compared from
                # the GPU's own root below, the gap reported
                n_unresolved += 1
                worst["P_unresolved"] = max(worst["P_unresolved"], e_p)
            # (2) from the root the GPU holds after the step
            sl, sr = blocks.side_state(b, 0), blocks.side_state(b, 1)

            def rect(st_, s_, p_):
                # the same codes as the root of (1) give the same rectified eigenvectors
                c0, sc0 = (new_root[(b, s_)][:2] if refresh else
                           (before[b][s_]["root_codes"], before[b][s_]["root_scales"]))
                if np.array_equal(st_["root_codes"], c0) and np.array_equal(st_["root_scales"], sc0):
                    return roots[s_][0]
                return o.rectified_eigenvectors(st_["root_codes"], st_["root_scales"], p_, k, 64, codebook)

            VL, VR = rect(sl, 0, m), rect(sr, 1, n)
            e_g = rel_fro(P_gpu, o.precondition_block(VL, sl["d"], VR, sr["d"], Gs[b]))
            assert e_g <= TOL, (label, t, b, "P from the GPU's root", e_g)
            worst["P_gpu_root"] = max(worst["P_gpu_root"], e_g)
            if root_cache:
                for s, V_, st_ in ((0, VL, sl), (1, VR, sr)):
                    Rt_gpu = blocks.view(b, s, BUF_ROOT_MAT).cpu().numpy()
                    e_r = rel_fro(Rt_gpu, o.root_matrix(V_, st_["d"]))
                    e_r2 = rel_fro(Rt_gpu, o.root_matrix(roots[s][0], roots[s][1])) if all_resolved else 0.0
                    assert e_r <= TOL and e_r2 <= TOL, (label, t, b, s, "root matrix", e_r, e_r2)
                    worst["root_mat"] = max(worst["root_mat"], e_r, e_r2)
    announce(f"step parity {label}: worst {worst}; codes differing from the oracle's own "
             f"{flips[0]} of {flips[1]}; block refreshes compared from the GPU's root (unresolved "
             f"eigenvalues or other codes) {n_unresolved}")
    blocks.close()
    return worst


def test_single_64x32_all_steps():
    require_gpu()
    wl = get_workload("single_64x32")
    _run_teacher_forced(wl.shapes, wl.gradients, wl.steps, beta=wl.beta, eps=wl.eps,
                        k=wl.bjorck_iters, root_interval=wl.root_interval, label="single_64x32")


def test_single_64x32_root_cache():
    require_gpu()
    wl = get_workload("single_64x32")
    _run_teacher_forced(wl.shapes, wl.gradients, 6, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                        root_interval=1, root_cache=True, label="single_64x32_cache")


@pytest.mark.parametrize("shapes,k,power_iters,T,cache", [
    ([(1, 1), (2, 3), (5, 1)], 1, 1, 1, False),           # degenerate tiny blocks
    ([(40, 72), (33, 33), (100, 7)], 2, 1, 2, True),      # ragged, across panels
    ([(96, 160), (130, 65)], 0, 2, 1, False),             # no Bjorck, two power steps
    ([(64, 64)], 5, 1, 1, True),
    ([(1100, 40)], 1, 1, 1, True),                        # panels taller than the register path
    ([(300, 257), (129, 128)], 1, 1, 1, False),           # ragged 128-column reflector blocks
])
@pytest.mark.parametrize("qr", ["auto", "blocked", "lookahead"])
def test_ragged_batches(shapes, k, power_iters, T, cache, qr):
    require_gpu()
    rng = np.random.default_rng(sum(m * 31 + n for m, n in shapes))
    scales = [(10.0 ** rng.uniform(-1, 1, (m, 1))) * (10.0 ** rng.uniform(-1, 1, (1, n))) for m, n in shapes]

    def grads(t):
        r = np.random.default_rng([t, len(shapes)])
        return [(r.standard_normal((m, n)) * sc).astype(np.float32) for (m, n), sc in zip(shapes, scales)]

    _run_teacher_forced(shapes, grads, 4, k=k, power_iters=power_iters, root_interval=T,
                        root_cache=cache, label=f"ragged {shapes} qr={qr}", qr=qr)


def test_blocked_qr_wide_outer_blocks():
    """Orders from 2048 take 256-column outer blocks in the blocked QR: a 2100-order side
    (eight full outer blocks and a ragged one of 52 columns) against the oracle."""
    require_gpu()
    shapes = [(2100, 300)]
    rng = np.random.default_rng(2100)
    scales = [(10.0 ** rng.uniform(-1, 1, (m, 1))) * (10.0 ** rng.uniform(-1, 1, (1, n))) for m, n in shapes]

    def grads(t):
        r = np.random.default_rng([t, 2100])
        return [(r.standard_normal((m, n)) * sc).astype(np.float32) for (m, n), sc in zip(shapes, scales)]

    _run_teacher_forced(shapes, grads, 3, k=1, power_iters=1, root_interval=1, root_cache=True,
                        label="blocked qr 2100", qr="blocked")


def test_single_1024_steps():
    """The 1024 x 1024 workload for its first root-refresh period (stats every step,
    root every 10 steps), so precondition runs with the identity root and then with
    a refreshed one."""
    require_gpu()
    wl = get_workload("single_1024")
    _run_teacher_forced(wl.shapes, wl.gradients, 11, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                        root_interval=wl.root_interval, label="single_1024")


@pytest.mark.parametrize("first,last", [(1, 25), (26, 50), (51, 75), (76, 100)])
def test_single_1024_bench_path(first, last):
    """The benchmark's configuration on the 1024 x 1024 workload over its whole
    schedule (100 steps, checked in four windows of 25): one shampoo4_step call per step
    with cached roots (the precondition runs beside the statistics update on 128 x 128
    tiles between refreshes), root every 10 steps (the statistics of the step after a
    refresh reuse the cached rectified eigenvectors), forced from the pre-step state."""
    require_gpu()
    wl = get_workload("single_1024")
    _run_teacher_forced(wl.shapes, wl.gradients, last, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                        root_interval=wl.root_interval, root_cache=True, use_step=True,
                        label=f"single_1024 bench path {first}-{last}", check_from=first)


def test_single_64x32_bench_path():
    """The 64 x 32 workload, all 20 steps, as the benchmark runs it (shampoo4_step,
    cached roots, root every step)."""
    require_gpu()
    wl = get_workload("single_64x32")
    _run_teacher_forced(wl.shapes, wl.gradients, wl.steps, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                        root_interval=wl.root_interval, root_cache=True, use_step=True,
                        label="single_64x32 bench path")


@pytest.mark.parametrize("shapes,T", [
    ([(40, 72), (33, 33), (100, 7)], 3),
    ([(300, 257), (129, 128)], 2),
])
def test_ragged_step_calls(shapes, T):
    """shampoo4_step with cached roots on ragged batches, forced from the pre-step state."""
    require_gpu()
    rng = np.random.default_rng(sum(m * 17 + n for m, n in shapes))
    scales = [(10.0 ** rng.uniform(-1, 1, (m, 1))) * (10.0 ** rng.uniform(-1, 1, (1, n))) for m, n in shapes]

    def grads(t):
        r = np.random.default_rng([t, 7, len(shapes)])
        return [(r.standard_normal((m, n)) * sc).astype(np.float32) for (m, n), sc in zip(shapes, scales)]

    _run_teacher_forced(shapes, grads, 2 * T + 1, root_interval=T, root_cache=True, use_step=True,
                        label=f"ragged step calls {shapes}")


def test_cnn_batch_two_steps():
    require_gpu()
    wl = get_workload("cnn_batch")
    sel = [0, 1, 2, 3, 4, 5, 6, 7]
    # a handful of the batch's blocks, every distinct shape represented
    shapes_all = wl.shapes
    seen, idx = set(), []
    for i, s in enumerate(shapes_all):
        if s not in seen:
            seen.add(s)
            idx.append(i)
    shapes = [shapes_all[i] for i in idx]

    def grads(t):
        return [wl.block_gradient(i, t) for i in idx]

    del sel
    _run_teacher_forced(shapes, grads, 2, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters, label="cnn_batch",
                        qr="blocked")


def test_dynamic_tree_single_64x32():
    """The dynamic tree codebook: every stage as with linear-square, codes bit-exact
    through the dynamic tree codec."""
    require_gpu()
    wl = get_workload("single_64x32")
    _run_teacher_forced(wl.shapes, wl.gradients, 8, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                        root_interval=2, root_cache=True, label="single_64x32 dt", codebook="dt")


@pytest.mark.parametrize("qr", ["auto", "blocked"])
def test_dynamic_tree_ragged(qr):
    require_gpu()
    shapes = [(40, 72), (1, 1), (130, 65), (257, 300)]
    rng = np.random.default_rng(77)
    scales = [(10.0 ** rng.uniform(-1, 1, (m, 1))) for m, n in shapes]

    def grads(t):
        r = np.random.default_rng([t, 77])
        return [(r.standard_normal((m, n)) * sc).astype(np.float32) for (m, n), sc in zip(shapes, scales)]

    _run_teacher_forced(shapes, grads, 3, k=1, root_interval=1, label=f"ragged dt qr={qr}", qr=qr,
                        codebook="dt")


def test_dynamic_tree_single_1024():
    require_gpu()
    wl = get_workload("single_1024")
    _run_teacher_forced(wl.shapes, wl.gradients, 3, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                        root_interval=2, label="single_1024 dt", codebook="dt")


def test_update_is_deterministic_and_resumable():
    """Two contexts fed the same gradients stay bit-identical; a context restarted from
    a saved state continues bit-identically."""
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    shapes = [(96, 64), (64, 130)]
    rng = np.random.default_rng(5)
    Gs = [[to_dev(rng.standard_normal(s).astype(np.float32)) for s in shapes] for _ in range(4)]
    cfg = Shampoo4Config(root_cache=True)
    announce("determinism/resume")
    a = Shampoo4Blocks(shapes, cfg)
    b = Shampoo4Blocks(shapes, cfg)
    for t in range(2):
        Pa = a.step(Gs[t], t + 1)
        Pb = b.step(Gs[t], t + 1)
        torch.cuda.synchronize()
        for x, y in zip(Pa, Pb):
            assert torch.equal(x, y)
    saved = a.state.clone()
    c = Shampoo4Blocks(shapes, cfg, state=saved)
    for t in range(2, 4):
        Pa = a.step(Gs[t], t + 1)
        Pc = c.step(Gs[t], t + 1)
        torch.cuda.synchronize()
        for x, y in zip(Pa, Pc):
            assert torch.equal(x, y)
    assert torch.equal(a.state, c.state)


def test_nonfinite_flag():
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks
    announce("nonfinite flag")
    blk = Shampoo4Blocks([(16, 8)])
    G = torch.zeros((16, 8), dtype=torch.float32, device="cuda")
    blk.update_stats([G])
    assert blk.check() == 0
    G[3, 2] = float("nan")
    blk.update_stats([G])
    assert blk.check() != 0
    assert blk.check() == 0      # cleared by the previous check


def _run_teacher_forced_fp32(shapes, grads_fn, steps, beta=0.95, eps=1e-6, k=1, root_interval=1,
                             label="", qr="auto"):
    """The 32-bit baseline (U kept in float32): same checks as the 4-bit path with the
    codec replaced by the identity on float32 values, so the new U must equal the GPU's
    own float32 Q bit for bit."""
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    cfg = Shampoo4Config(beta=beta, eps=eps, bjorck_iters=k, fp32_state=True, qr_schedule=qr)
    announce(f"fp32 state {label}: init {shapes}")
    blocks = Shampoo4Blocks(shapes, cfg)
    torch.cuda.synchronize()
    for b, (m, n) in enumerate(shapes):
        for s, p in ((0, m), (1, n)):
            assert np.array_equal(blocks.eigenvectors(b, s).cpu().numpy(), np.eye(p, dtype=np.float32))
            assert np.array_equal(blocks.eigenvectors(b, s, root=True).cpu().numpy(), np.eye(p, dtype=np.float32))
    for t in range(1, steps + 1):
        Gs = grads_fn(t)
        Gd = [to_dev(G) for G in Gs]
        before = [[(blocks.eigenvectors(b, s).cpu().numpy(), blocks.side_state(b, s)["lam"]) for s in (0, 1)]
                  for b in range(len(shapes))]
        announce(f"fp32 state {label}: t={t} update_stats")
        blocks.update_stats(Gd)
        torch.cuda.synchronize()
        for b, (m, n) in enumerate(shapes):
            for s, p in ((0, m), (1, n)):
                U0, lam0 = before[b][s]
                V = o.bjorck(U0.astype(np.float64), k)
                Lt_ref = o.statistics(V, lam0, o.side_gradient(Gs[b], s), beta)
                Lt_gpu = blocks.view(b, s, 17).cpu().numpy().astype(np.float64)
                assert rel_fro(Lt_gpu, Lt_ref) <= TOL, (label, t, b, s, "statistic")
                Q_ref, lam_ref = o.eigen_refresh(Lt_gpu, V, 1)
                Q32 = blocks.view(b, s, 18).cpu().numpy()
                lam_gpu = blocks.side_state(b, s)["lam"].astype(np.float64)
                Qg = Q32.astype(np.float64)
                assert rel_fro((Qg * lam_gpu) @ Qg.T, (Q_ref * lam_ref) @ Q_ref.T) <= TOL, (label, t, b, s)
                assert rel_fro(lam_gpu, lam_ref) <= TOL, (label, t, b, s, "eigenvalues")
                assert np.array_equal(blocks.eigenvectors(b, s).cpu().numpy().view(np.uint32), Q32.view(np.uint32))
        if t % root_interval == 0:
            blocks.refresh_root()
            torch.cuda.synchronize()
            for b in range(len(shapes)):
                for s in (0, 1):
                    assert torch.equal(blocks.eigenvectors(b, s, root=True), blocks.eigenvectors(b, s))
        announce(f"fp32 state {label}: t={t} precondition")
        outs = blocks.precondition(Gd)
        torch.cuda.synchronize()
        for b, (m, n) in enumerate(shapes):
            sl, sr = blocks.side_state(b, 0), blocks.side_state(b, 1)
            VL = o.bjorck(blocks.eigenvectors(b, 0, root=True).cpu().numpy().astype(np.float64), k)
            VR = o.bjorck(blocks.eigenvectors(b, 1, root=True).cpu().numpy().astype(np.float64), k)
            P_ref = o.precondition_block(VL, sl["d"], VR, sr["d"], Gs[b])
            assert rel_fro(outs[b].cpu().numpy(), P_ref) <= TOL, (label, t, b, "P")
    assert blocks.check() == 0
    blocks.close()


@pytest.mark.parametrize("qr", ["auto", "blocked"])
def test_fp32_state_ragged(qr):
    require_gpu()
    shapes = [(40, 72), (130, 65), (1, 3)]
    rng = np.random.default_rng(21)
    scales = [(10.0 ** rng.uniform(-1, 1, (m, 1))) * (10.0 ** rng.uniform(-1, 1, (1, n))) for m, n in shapes]

    def grads(t):
        r = np.random.default_rng([t, 99])
        return [(r.standard_normal((m, n)) * sc).astype(np.float32) for (m, n), sc in zip(shapes, scales)]

    _run_teacher_forced_fp32(shapes, grads, 3, root_interval=2, label=f"ragged qr={qr}", qr=qr)


def test_fp32_state_single_1024():
    require_gpu()
    wl = get_workload("single_1024")
    _run_teacher_forced_fp32(wl.shapes, wl.gradients, 3, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                             root_interval=1, label="single_1024")


def test_blocked_parameter_views():
    """Blocks of real parameters as strided views (no copies): the step reads them with
    their leading dimensions and writes the directions into views of a full-size buffer;
    the result equals the same step on contiguous copies, bit for bit."""
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks, blocking
    announce("blocked parameter views")
    rng = np.random.default_rng(4)
    params = [torch.from_numpy(rng.standard_normal((1100, 70)).astype(np.float32)).cuda(),
              torch.from_numpy(rng.standard_normal((16, 8, 3, 3)).astype(np.float32)).cuda()]
    plans = blocking.plan_blocks([p.shape for p in params])
    shapes = blocking.block_shapes(plans)
    assert shapes == [(1024, 70), (76, 70), (16, 72)]
    views = blocking.block_views(params, plans)
    dirs = [torch.empty_like(p) for p in params]
    out_views = blocking.block_views(dirs, plans)
    a = Shampoo4Blocks(shapes)
    a.step(views, 1, outs=out_views)
    b = Shampoo4Blocks(shapes)
    ref = b.step([v.contiguous() for v in views], 1)
    torch.cuda.synchronize()
    for o, r in zip(out_views, ref):
        assert torch.equal(o, r)
    a.close()
    b.close()


@pytest.mark.parametrize("qr", ["auto", "lookahead", "blocked"])
def test_graph_replays_match_eager(qr):
    """update_stats replayed from a captured HIP graph (several replays, with host reads
    and synchronizations between them, both the cached-eigenvector variant and the plain
    one) leaves the state bit-identical to eager launches."""
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    shapes = [(96, 64), (130, 200)]
    rng = np.random.default_rng(9)
    Gs = [[to_dev(rng.standard_normal(s).astype(np.float32)) for s in shapes] for _ in range(5)]
    announce(f"graph replays qr={qr}")
    eager = Shampoo4Blocks(shapes, Shampoo4Config(root_cache=True, qr_schedule=qr))
    graph = Shampoo4Blocks(shapes, Shampoo4Config(root_cache=True, qr_schedule=qr, graphs=True))
    for t in range(5):
        root_interval = 2   # alternates the two captured variants
        Pe = eager.step(Gs[t], t + 1, root_interval)
        Pg = graph.step(Gs[t], t + 1, root_interval)
        torch.cuda.synchronize()
        for b in range(len(shapes)):      # the state's alignment padding is never written
            for s_ in (0, 1):
                se, sg = eager.side_state(b, s_), graph.side_state(b, s_)
                for k in se:
                    assert np.array_equal(se[k], sg[k]), (qr, t, b, s_, k)
        for a, b in zip(Pe, Pg):
            assert torch.equal(a, b), (qr, t, "P")
    eager.close()
    graph.close()


def test_graph_replays_follow_operand_alignment():
    """A graph captured while the gradients allowed 16-byte loads is not replayed for a
    call whose gradient is a view with a leading dimension that is not a multiple of 4
    (the vector-load kernels would break their precondition): the state and P stay
    bit-identical to eager launches on the same sequence of calls."""
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    shapes = [(96, 64), (130, 200)]
    rng = np.random.default_rng(10)
    aligned = [[to_dev(rng.standard_normal(s).astype(np.float32)) for s in shapes] for _ in range(3)]
    wide = [[to_dev(rng.standard_normal((m, n + 3)).astype(np.float32)) for (m, n) in shapes] for _ in range(3)]
    views = [[w[:, 1:n + 1] for w, (m, n) in zip(ws, shapes)] for ws in wide]   # ld = n + 3, offset 4 B
    seq = [aligned[0], views[0], aligned[1], views[1], views[2], aligned[2]]
    announce("graph replays across operand alignment")
    eager = Shampoo4Blocks(shapes, Shampoo4Config(root_cache=True))
    graph = Shampoo4Blocks(shapes, Shampoo4Config(root_cache=True, graphs=True))
    for t, G in enumerate(seq, start=1):
        Pe = eager.step(G, t, 2)
        Pg = graph.step(G, t, 2)
        torch.cuda.synchronize()
        for b in range(len(shapes)):
            for s_ in (0, 1):
                se, sg = eager.side_state(b, s_), graph.side_state(b, s_)
                for k in se:
                    assert np.array_equal(se[k], sg[k]), (t, b, s_, k)
        for a, b in zip(Pe, Pg):
            assert torch.equal(a, b), (t, "P")
    eager.close()
    graph.close()


def test_step_call_matches_separate_calls_1024():
    """The one-call step against the three calls on the 1024 x 1024 block (the fused QR
    schedule with the precondition beside it), bit for bit over steps with and without a
    refresh."""
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    wl = get_workload("single_1024")
    announce("step call vs separate calls 1024")
    one = Shampoo4Blocks(wl.shapes, Shampoo4Config(root_cache=True))
    sep = Shampoo4Blocks(wl.shapes, Shampoo4Config(root_cache=True))
    for t in range(1, 6):
        G = [to_dev(g) for g in wl.gradients(t)]
        P1 = one.step(G, t, root_interval=2)
        sep.update_stats(G)
        if t % 2 == 0:
            sep.refresh_root()
        P2 = sep.precondition(G)
        torch.cuda.synchronize()
        assert torch.equal(P1[0], P2[0]), (t, "P")
        for s_ in (0, 1):
            s1, s2 = one.side_state(0, s_), sep.side_state(0, s_)
            for k in s1:
                assert np.array_equal(s1[k], s2[k]), (t, s_, k)
    one.close()
    sep.close()


@pytest.mark.parametrize("qr", ["auto", "blocked"])
def test_step_call_matches_separate_calls(qr):
    """shampoo4_step (precondition beside the statistics update on a second stream when
    no refresh is due) leaves the state and P bit-identical to update_stats,
    refresh_root and precondition called one after another on one stream, over steps
    with and without a refresh, with and without cached roots."""
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    shapes = [(96, 64), (130, 200), (512, 384)]
    rng = np.random.default_rng(21)
    Gs = [[to_dev(rng.standard_normal(s).astype(np.float32)) for s in shapes] for _ in range(7)]
    for cache in (True, False):
        announce(f"step call vs separate calls qr={qr} root_cache={cache}")
        one = Shampoo4Blocks(shapes, Shampoo4Config(root_cache=cache, qr_schedule=qr))
        sep = Shampoo4Blocks(shapes, Shampoo4Config(root_cache=cache, qr_schedule=qr))
        for t in range(1, 8):
            P1 = one.step(Gs[t - 1], t, root_interval=3)
            sep.update_stats(Gs[t - 1])
            if t % 3 == 0:
                sep.refresh_root()
            P2 = sep.precondition(Gs[t - 1])
            torch.cuda.synchronize()
            for b in range(len(shapes)):
                assert torch.equal(P1[b], P2[b]), (qr, cache, t, b, "P")
                for s_ in (0, 1):
                    s1, s2 = one.side_state(b, s_), sep.side_state(b, s_)
                    for k in s1:
                        assert np.array_equal(s1[k], s2[k]), (qr, cache, t, b, s_, k)
        one.close()
        sep.close()


# ---------------------------------------------------------------------------
# The float64 statistics update (SHAMPOO4_FLAG_FP64_REFRESH)
# ---------------------------------------------------------------------------

def test_fp64_refresh_single_64x32_all_steps():
    """The 64 x 32 workload (rank-deficient on its 64 side for the first step) over its 20
    steps with the float64 update, as the benchmark runs it; float64 resolves eigenvalues
    down to about p 2^-53 lam_max, so the whole step is compared from the pre-step state
    wherever the codes agree."""
    require_gpu()
    wl = get_workload("single_64x32")
    w = _run_teacher_forced(wl.shapes, wl.gradients, wl.steps, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                            root_interval=wl.root_interval, root_cache=True, use_step=True, fp64=True,
                            label="single_64x32 fp64")
    # the statistic to float64 rounding; d from the pre-step state to about float32's
    # storage of the eigenvalues (float32 refreshes: within 1e-3 plus the floor's bound)
    assert w["stat"] <= 1e-12 and w["d"] <= 1e-5, w


@pytest.mark.parametrize("shapes,k,T", [
    ([(1, 1), (2, 3), (5, 1)], 1, 1),
    ([(40, 72), (33, 33), (100, 7)], 2, 2),
    ([(1100, 40)], 1, 1),
    ([(300, 257), (129, 128)], 0, 1),
])
def test_fp64_refresh_ragged(shapes, k, T):
    require_gpu()
    rng = np.random.default_rng(sum(m * 13 + n for m, n in shapes))
    scales = [(10.0 ** rng.uniform(-1, 1, (m, 1))) * (10.0 ** rng.uniform(-1, 1, (1, n))) for m, n in shapes]

    def grads(t):
        r = np.random.default_rng([t, 64, len(shapes)])
        return [(r.standard_normal((m, n)) * sc).astype(np.float32) for (m, n), sc in zip(shapes, scales)]

    w = _run_teacher_forced(shapes, grads, 4, k=k, root_interval=T, root_cache=True, use_step=True, fp64=True,
                            label=f"fp64 ragged {shapes}")
    assert w["stat"] <= 1e-12, w


def test_fp64_refresh_single_1024():
    require_gpu()
    wl = get_workload("single_1024")
    w = _run_teacher_forced(wl.shapes, wl.gradients, 11, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                            root_interval=wl.root_interval, root_cache=True, use_step=True, fp64=True,
                            label="single_1024 fp64")
    assert w["stat"] <= 1e-12, w
