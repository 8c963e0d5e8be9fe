"""GPU parity of the diagonal fallback ("Shampoo -- Second-Order Optimizer", "Blocked and
distributed variants": a side over the size threshold drops its factor and keeps
diagonal AdaGrad along it) against the oracle, teacher-forced from the GPU's pre-step
state: the diagonal statistic of every diagonal side, the full sides of one-sided
blocks (statistic, Q diag(lam) Q^T, eigenvalues, codes bit-exact through the codec on
the GPU's own Q), d at every refresh, and the preconditioned gradient from the root the
GPU holds (rel-Frobenius <= 1e-3)."""

import numpy as np
import pytest
import torch

from oracle import codec
from oracle import shampoo4 as o
from tests.gpu_util import announce, rel_fro, require_gpu, to_dev

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _grads(shapes, seed):
    rng = np.random.default_rng(seed)
    scales = [(10.0 ** rng.uniform(-1, 1, (m, 1))) * (10.0 ** rng.uniform(-1, 1, (1, n))) for m, n in shapes]

    def grads(t):
        r = np.random.default_rng([seed, t])
        return [(r.standard_normal((m, n)) * sc).astype(np.float32) for (m, n), sc in zip(shapes, scales)]

    return grads


def _oracle_from_gpu(blocks, shapes, diagonal, beta, eps, k):
    orc = o.Shampoo4Oracle(shapes, beta=beta, eps=eps, bjorck_iters=k, diagonal=diagonal)
    for b in range(len(shapes)):
        for s in (0, 1):
            st = blocks.side_state(b, s)
            side = orc.sides[b][s]
            side.codes, side.scales, side.lam = st["codes"], st["scales"], st["lam"]
            side.root_codes, side.root_scales, side.d = st["root_codes"], st["root_scales"], st["d"]
    return orc


def _run(shapes, diagonal, steps, T=1, root_cache=False, use_step=False, k=1, beta=0.95, eps=1e-6, label=""):
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    cfg = Shampoo4Config(beta=beta, eps=eps, bjorck_iters=k, root_cache=root_cache)
    announce(f"diag {label}: init {shapes} {diagonal}")
    blocks = Shampoo4Blocks(shapes, cfg, diagonal=diagonal)
    torch.cuda.synchronize()
    for b, (m, n) in enumerate(shapes):
        for s, p in ((0, m), (1, n)):
            st = blocks.side_state(b, s)
            assert np.all(st["lam"] == 0) and np.all(st["d"] == 1)
            if diagonal[b][s]:
                assert st["codes"].size == 0 and st["scales"].size == 0
    grads = _grads(shapes, sum(m + 3 * n for m, n in shapes))
    worst = {"diag_lam": 0.0, "stat": 0.0, "recon": 0.0, "P": 0.0}
    for t in range(1, steps + 1):
        Gs = grads(t)
        Gd = [to_dev(G) for G in Gs]
        refresh = t % T == 0
        before = [[blocks.side_state(b, s) for s in (0, 1)] for b in range(len(shapes))]
        announce(f"diag {label}: t={t}")
        if use_step:
            outs = blocks.step(Gd, t, T)
        else:
            blocks.update_stats(Gd)
            if refresh:
                blocks.refresh_root()
            outs = blocks.precondition(Gd)
        torch.cuda.synchronize()
        for b, (m, n) in enumerate(shapes):
            for s, p in ((0, m), (1, n)):
                st0 = before[b][s]
                after = blocks.side_state(b, s)
                Gside = o.side_gradient(Gs[b], s)
                if diagonal[b][s]:
                    ref = o.diagonal_statistics(st0["lam"], Gside, beta)
                    e = float(np.max(np.abs(after["lam"] / ref - 1.0)))
                    assert e <= 1e-4, (label, t, b, s, "diagonal statistic", e)
                    worst["diag_lam"] = max(worst["diag_lam"], e)
                else:
                    V = o.rectified_eigenvectors(st0["codes"], st0["scales"], p, k)
                    Lt_ref = o.statistics(V, st0["lam"], Gside, beta)
                    Lt_gpu = blocks.view(b, s, 17).cpu().numpy().astype(np.float64)
                    e_stat = rel_fro(Lt_gpu, Lt_ref)
                    assert e_stat <= TOL, (label, t, b, s, "statistic", e_stat)
                    Q_ref, lam_ref = o.eigen_refresh(Lt_ref, V)
                    Q32 = blocks.view(b, s, 18).cpu().numpy()
                    Qg = Q32.astype(np.float64)
                    lam_g = after["lam"].astype(np.float64)
                    e_rec = rel_fro((Qg * lam_g) @ Qg.T, (Q_ref * lam_ref) @ Q_ref.T)
                    assert e_rec <= TOL, (label, t, b, s, "Q diag(lam) Q^T", e_rec)
                    assert rel_fro(lam_g, lam_ref) <= TOL, (label, t, b, s, "eigenvalues")
                    c_ref, s_ref = codec.quantize_matrix(Q32, 64)
                    assert np.array_equal(after["codes"], c_ref), (label, t, b, s, "codes")
                    assert np.array_equal(after["scales"].view(np.uint32), s_ref.view(np.uint32))
                    worst["stat"] = max(worst["stat"], e_stat)
                    worst["recon"] = max(worst["recon"], e_rec)
                if refresh:
                    assert np.allclose(after["d"], o.root_scaling(after["lam"], eps), rtol=2e-6, atol=0), \
                        (label, t, b, s, "d")
                    if not diagonal[b][s]:
                        assert np.array_equal(after["root_codes"], after["codes"])
                else:
                    assert np.array_equal(after["d"], st0["d"]), (label, t, b, s, "d changed without a refresh")
        orc = _oracle_from_gpu(blocks, shapes, diagonal, beta, eps, k)
        P_ref = orc.precondition(Gs)
        for b in range(len(shapes)):
            P = outs[b].cpu().numpy()
            assert np.all(np.isfinite(P))
            e_p = rel_fro(P, P_ref[b])
            assert e_p <= TOL, (label, t, b, "P", e_p)
            worst["P"] = max(worst["P"], e_p)
    assert blocks.check() == 0
    announce(f"diag {label}: worst {worst}")
    blocks.close()
    return worst


@pytest.mark.parametrize("root_cache,use_step,T", [(False, False, 1), (True, False, 2), (True, True, 2),
                                                   (False, True, 1)])
def test_mixed_batch(root_cache, use_step, T):
    """One-sided blocks of both orientations, a both-diagonal block, a plain block and a
    degenerate both-diagonal column in one batch."""
    shapes = [(64, 2000), (40, 72), (300, 96), (70, 50), (33, 1)]
    diagonal = [(False, True), (False, False), (True, False), (True, True), (True, True)]
    _run(shapes, diagonal, 5, T=T, root_cache=root_cache, use_step=use_step,
         label=f"mixed cache={root_cache} step={use_step} T={T}")


def test_one_sided_tall_and_wide_panels():
    """Kept sides across register and global panels: order 1100 (taller than the register
    panel) with a diagonal side of 5000, and a diagonal side of order 9000 (above the
    limit of a side with eigenvectors)."""
    shapes = [(1100, 5000), (9000, 300)]
    diagonal = [(False, True), (True, False)]
    _run(shapes, diagonal, 3, T=1, root_cache=True, use_step=True, label="tall and wide")


@pytest.mark.timeout(300)
def test_vocabulary_sized_block():
    """A [1024, 32768] block (the blog's vocabulary-sized example, n = 32768) with its
    32768 side diagonal and the 1024 side kept in 4 bits, as blocking without tiling and a
    threshold of 8192 plans it."""
    from bit_quantized_shampoo_amd import blocking
    plans = blocking.plan_blocks([(1024, 32768)], block=None, max_dim=8192)
    shapes, diagonal = blocking.block_shapes(plans), blocking.block_diagonal_sides(plans)
    assert shapes == [(1024, 32768)] and diagonal == [(False, True)]
    _run(shapes, diagonal, 3, T=1, root_cache=True, use_step=True, label="vocabulary")
