"""Teacher-forced parity of the whole step against the CPU oracle.

Each entry point is checked from the state the GPU itself produced:
  update_stats   the oracle recomputes the rectified eigenvectors from the GPU's
                 codes, the statistic from them and the GPU's eigenvalues, and the
                 refresh from the GPU's statistic; compared are the statistic, the
                 basis-invariant product Q diag(lam) Q^T and the eigenvalues
                 (rel-Frobenius <= 1e-3), and the new codes, which must equal the
                 oracle codec applied to the GPU's own fp32 Q bit for bit;
  refresh_root   d and the root codes;
  precondition   the oracle's preconditioned gradient from the GPU's root state
                 (rel-Frobenius <= 1e-3).
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


def _run_teacher_forced(shapes, grads_fn, steps, beta=0.95, eps=1e-6, k=1, power_iters=1,
                        root_interval=1, root_cache=False, label="", qr="auto", codebook="ls",
                        sample=None, all_sides=None):
    """`sample`: the blocks checked against the oracle (default: every block).
    `all_sides(blocks, t)`: an optional extra check after each update_stats."""
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    cfg = Shampoo4Config(beta=beta, eps=eps, bjorck_iters=k, power_iters=power_iters,
                         root_cache=root_cache, qr_schedule=qr, codebook=codebook)
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
    worst = {"stat": 0.0, "recon": 0.0, "lam": 0.0, "P": 0.0}
    for t in range(1, steps + 1):
        Gs = grads_fn(t)
        Gd = [to_dev(G) for G in Gs]
        before = {b: [blocks.side_state(b, s) for s in (0, 1)] for b in checked}
        announce(f"step parity {label}: t={t} update_stats")
        blocks.update_stats(Gd)
        torch.cuda.synchronize()
        if all_sides is not None:
            all_sides(blocks, t)
        for b in checked:
            m, n = shapes[b]
            for s, p in ((0, m), (1, n)):
                st = before[b][s]
                Gs_side = o.side_gradient(Gs[b], s)
                V = o.rectified_eigenvectors(st["codes"], st["scales"], p, k, 64, codebook)
                Lt_ref = o.statistics(V, st["lam"], Gs_side, beta)
                Lt_gpu = blocks.view(b, s, 17).cpu().numpy().astype(np.float64)
                # symmetric up to the float32 rounding of the K-scaled products (off-diagonal
                # tiles are stored mirrored)
                assert rel_fro(Lt_gpu, Lt_gpu.T) <= 1e-6, (label, t, b, s, "statistic not symmetric")
                e_stat = rel_fro(Lt_gpu, Lt_ref)
                assert e_stat <= TOL, (label, t, b, s, "statistic", e_stat)
                Q_ref, lam_ref = o.eigen_refresh(Lt_gpu, V, power_iters)
                Q_gpu32 = blocks.view(b, s, 18).cpu().numpy()
                after = blocks.side_state(b, s)
                lam_gpu = after["lam"].astype(np.float64)
                Q_gpu = Q_gpu32.astype(np.float64)
                e_rec = rel_fro((Q_gpu * lam_gpu) @ Q_gpu.T, (Q_ref * lam_ref) @ Q_ref.T)
                e_lam = rel_fro(lam_gpu, lam_ref)
                assert e_rec <= TOL, (label, t, b, s, "Q diag(lam) Q^T", e_rec)
                assert e_lam <= TOL, (label, t, b, s, "eigenvalues", e_lam)
                assert np.allclose(Q_gpu.T @ Q_gpu, np.eye(p), atol=1e-4), (label, t, b, s, "orthonormal Q")
                c_ref, s_ref = codec.quantize_matrix(Q_gpu32, 64, codebook)
                assert np.array_equal(after["codes"], c_ref), (label, t, b, s, "codes")
                assert np.array_equal(after["scales"].view(np.uint32), s_ref.view(np.uint32))
                worst["stat"] = max(worst["stat"], e_stat)
                worst["recon"] = max(worst["recon"], e_rec)
                worst["lam"] = max(worst["lam"], e_lam)
        if t % root_interval == 0:
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
        announce(f"step parity {label}: t={t} precondition")
        outs = blocks.precondition(Gd)
        torch.cuda.synchronize()
        for P in outs:
            assert bool(torch.isfinite(P).all()), (label, t, "non-finite preconditioned gradient")
        for b in checked:
            m, n = shapes[b]
            sl, sr = blocks.side_state(b, 0), blocks.side_state(b, 1)
            VL = o.rectified_eigenvectors(sl["root_codes"], sl["root_scales"], m, k, 64, codebook)
            VR = o.rectified_eigenvectors(sr["root_codes"], sr["root_scales"], n, k, 64, codebook)
            P_ref = o.precondition_block(VL, sl["d"], VR, sr["d"], Gs[b])
            e_p = rel_fro(outs[b].cpu().numpy(), P_ref)
            assert e_p <= TOL, (label, t, b, "P", e_p)
            worst["P"] = max(worst["P"], e_p)
    announce(f"step parity {label}: worst {worst}")
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


def test_single_1024_steps():
    """The 1024 x 1024 workload for its first root-refresh period (stats every step,
    root every 10 steps), so precondition runs with the identity root and then with
    a refreshed one."""
    require_gpu()
    wl = get_workload("single_1024")
    _run_teacher_forced(wl.shapes, wl.gradients, 11, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                        root_interval=wl.root_interval, label="single_1024")


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
