"""Grafting epilogue on the GPU against the oracle ("Shampoo -- Second-Order Optimizer",
section "Grafting: borrow a step size that already works").

Same seeded W, G, P on both sides (teacher-forced: every step starts from the GPU's own
float32 W and moments).  Per element, |W_gpu - W_ref| <= 1e-5 |lr s P| + ulp(W_ref): the
block scale s carries float32 norms over up to 1M elements (relative error well under
1e-5 against float64), and the update itself is one fused multiply-add rounded once to
float32.  The Adam moments (beta x + (1 - beta) y) are compared elementwise within 1e-6 of
beta |x| + (1 - beta) |y|.  Shapes
cover several row tiles, a ragged last tile and rows longer than one workgroup's tile."""

import numpy as np
import pytest
import torch

from oracle import graft as og
from tests.gpu_util import announce, rel_fro, require_gpu, to_dev

pytestmark = pytest.mark.gpu

SHAPES = [(64, 32), (33, 70), (1024, 1024), (5, 4100)]
TOL = 1e-5


def _inputs(shapes, seed):
    rng = np.random.default_rng(seed)
    W = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    G = [(rng.standard_normal(s) * 10.0 ** rng.uniform(-2, 2)).astype(np.float32) for s in shapes]
    P = [(rng.standard_normal(s) * 10.0 ** rng.uniform(-3, 3)).astype(np.float32) for s in shapes]
    return W, G, P


@pytest.mark.parametrize("mode", ["sgd", "adam"])
def test_graft_matches_oracle(mode):
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks
    announce(f"graft {mode} {SHAPES}")
    blk = Shampoo4Blocks(SHAPES)
    W, _, _ = _inputs(SHAPES, 1)
    Wd = [to_dev(w) for w in W]
    Md = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in SHAPES]
    Vd = [torch.zeros(s, dtype=torch.float32, device="cuda") for s in SHAPES]
    # the ABI takes float32 parameters: the oracle gets the same float32 values
    prm = {k: float(np.float32(v)) for k, v in
           dict(lr=0.05, eps_graft=1e-6, beta1=0.9, beta2=0.99, eps_adam=1e-8).items()}
    for t in range(1, 4):
        _, G, P = _inputs(SHAPES, 10 + t)
        # teacher forcing: the oracle starts each step from the GPU's own state
        W_before = [w.cpu().numpy().astype(np.float64) for w in Wd]
        Mr = [m.cpu().numpy().astype(np.float64) for m in Md]
        Vr = [v.cpu().numpy().astype(np.float64) for v in Vd]
        blk.graft([to_dev(g) for g in G], [to_dev(p) for p in P], Wd,
                  list(zip(Md, Vd)) if mode == "adam" else None, mode=mode, step=t, **prm)
        torch.cuda.synchronize()
        for b in range(len(SHAPES)):
            Wn, Mn, Vn, s = og.graft_step(W_before[b], G[b], P[b], mode=og.ADAM if mode == "adam" else og.SGD,
                                          t=t, m=Mr[b], v=Vr[b], **prm)
            got = Wd[b].cpu().numpy().astype(np.float64)
            upd = np.abs(Wn - W_before[b])
            ulp = np.spacing(np.abs(Wn).astype(np.float32)).astype(np.float64)
            excess = np.abs(got - Wn) - (TOL * upd + ulp)
            assert np.all(excess <= 0), (mode, t, SHAPES[b], "W update", float(excess.max()))
            assert rel_fro(got - W_before[b], Wn - W_before[b]) <= 1e-3
            if mode == "adam":
                # each moment is beta x + (1 - beta) y in float32: a few roundings of the
                # larger term, which can exceed the result itself when the terms cancel
                g64 = G[b].astype(np.float64)
                for dev, ref, prev, y, beta, nm in ((Md[b], Mn, Mr[b], g64, prm["beta1"], "M"),
                                                    (Vd[b], Vn, Vr[b], g64 * g64, prm["beta2"], "V")):
                    d = dev.cpu().numpy().astype(np.float64)
                    scale = beta * np.abs(prev) + (1 - beta) * np.abs(y)
                    excess = np.abs(d - ref) - 1e-6 * scale
                    assert np.all(excess <= 1e-38), (t, SHAPES[b], nm, float(excess.max()))
    assert blk.check() == 0
    blk.close()


def test_graft_deterministic_and_after_precondition():
    """The grafted update of the step's own preconditioned direction, twice from the same
    state: bit-identical."""
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks
    shapes = [(96, 64), (64, 130)]
    announce(f"graft after precondition {shapes}")
    rng = np.random.default_rng(3)
    G = [to_dev(rng.standard_normal(s).astype(np.float32)) for s in shapes]
    W0 = [rng.standard_normal(s).astype(np.float32) for s in shapes]
    outs = []
    for _ in range(2):
        blk = Shampoo4Blocks(shapes)
        P = blk.step(G, 1)
        W = [to_dev(w) for w in W0]
        blk.graft(G, P, W, mode="sgd", lr=0.1)
        torch.cuda.synchronize()
        outs.append([w.cpu().numpy() for w in W])
        # the update direction is P's, with the SGD norm
        for b in range(len(shapes)):
            step = W0[b].astype(np.float64) - outs[-1][b]
            Pn = P[b].cpu().numpy().astype(np.float64)
            want = 0.1 * np.linalg.norm(G[b].cpu().numpy()) / (np.linalg.norm(Pn) + 1e-8) * Pn
            assert rel_fro(step, want) <= TOL
        blk.close()
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_graft_rejects_bad_arguments():
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks
    from bit_quantized_shampoo_amd._lib import Shampoo4Error
    announce("graft argument checks")
    blk = Shampoo4Blocks([(8, 4)])
    G = [torch.zeros((8, 4), device="cuda")]
    P = [torch.zeros((8, 4), device="cuda")]
    W = [torch.zeros((8, 4), device="cuda")]
    with pytest.raises(ValueError):
        blk.graft(G, P, W, mode="adam", moments=None, step=1)   # Adam without moments
    with pytest.raises(Shampoo4Error):
        M = [(torch.zeros((8, 4), device="cuda"), torch.zeros((8, 4), device="cuda"))]
        blk.graft(G, P, W, M, mode="adam", step=0)              # step must be >= 1
    with pytest.raises(ValueError):
        blk.graft(G, P, W, mode="rmsprop")
    blk.close()
