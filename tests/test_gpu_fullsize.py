"""Parity at the workloads' full sizes, in the configuration bench.py times (every block
of the batch on the GPU, cached root matrices, the automatic QR schedule, the workload's
Bjorck iterations and root interval).

The oracle is too slow for every block of these batches, so:
  * sampled blocks (every distinct shape of the CNN batch and its last block, a block
    of each layer kind of the transformer batch's first layer and its last block, the
    first and last 4096 blocks of the stress batch) get the full teacher-forced
    comparison of the step harness (statistic, Q diag(lam) Q^T, eigenvalues, codes, d,
    root matrices, preconditioned gradient) over the workload's whole schedule (10, 10
    and 3 steps, checked in windows, one test each; the 4096 batch's last step also on
    its last block), every step run as one shampoo4_step call like the benchmark;
  * every side gets the checks that hold at any size: the new Q is orthonormal
    (computed in float64 on the device), finite, and a seeded sample of sides has codes
    equal, bit for bit, to the oracle codec applied to the GPU's own float32 Q.
"""

import numpy as np
import pytest
import torch

from oracle import codec
from tests.gpu_util import announce, require_gpu
from tests.test_gpu_step import _run_teacher_forced
from workloads import get_workload

pytestmark = pytest.mark.gpu


def _side_checks(shapes, ncodes, seed):
    rng = np.random.default_rng(seed)
    sides = [(b, s) for b in range(len(shapes)) for s in (0, 1)]
    pick = sorted(rng.choice(len(sides), size=min(ncodes, len(sides)), replace=False).tolist())

    def check(blocks, t):
        worst = 0.0
        for b, s in sides:
            Q = blocks.view(b, s, 18)
            assert bool(torch.isfinite(Q).all()), (t, b, s, "non-finite Q")
            Qd = Q.double()
            e = float((Qd.T @ Qd - torch.eye(Q.shape[0], dtype=torch.float64, device=Q.device)).abs().max())
            worst = max(worst, e)
            assert e <= 1e-4, (t, b, s, "Q not orthonormal", e)
        for i in pick:
            b, s = sides[i]
            Q32 = blocks.view(b, s, 18).cpu().numpy()
            st = blocks.side_state(b, s)
            c_ref, s_ref = codec.quantize_matrix(Q32, 64)
            assert np.array_equal(st["codes"], c_ref), (t, b, s, "codes")
            assert np.array_equal(st["scales"].view(np.uint32), s_ref.view(np.uint32)), (t, b, s, "scales")
        announce(f"  all {len(sides)} sides orthonormal (worst {worst:.2e}), codes of {len(pick)} sides bit-exact")

    return check


def _distinct_shape_blocks(shapes):
    seen, idx = set(), []
    for i, sh in enumerate(shapes):
        if sh not in seen:
            seen.add(sh)
            idx.append(i)
    return idx


@pytest.mark.timeout(600)
@pytest.mark.parametrize("name,first,last,blocks,ncodes", [
    ("cnn_batch", 1, 5, "sample", 64),
    ("cnn_batch", 6, 10, "sample", 64),
    ("transformer_batch", 1, 5, "sample", 24),
    ("transformer_batch", 6, 10, "sample", 24),
    ("large_4096", 1, 2, "first", 6),
    ("large_4096", 3, 3, "first", 6),
    ("large_4096", 3, 3, "last", 6),
])
def test_full_size_sampled(name, first, last, blocks, ncodes):
    require_gpu()
    wl = get_workload(name)
    shapes = wl.shapes
    if name == "cnn_batch":
        sample = sorted(set(_distinct_shape_blocks(shapes) + [len(shapes) - 1]))
    elif name == "transformer_batch":
        # one block of each of the four layer kinds in the first layer, and the last block
        sample = [0, 3, 4, 8, len(shapes) - 1]
    else:
        sample = [0] if blocks == "first" else [len(shapes) - 1]
    announce(f"full size {name}: {len(shapes)} blocks, oracle on blocks {sample}, steps {first}-{last}")
    _run_teacher_forced(shapes, wl.gradients, last, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                        power_iters=wl.power_iters, root_interval=wl.root_interval, root_cache=True,
                        label=f"{name} {first}-{last}", qr="auto", sample=sample, use_step=True,
                        check_from=first, all_sides=_side_checks(shapes, ncodes, seed=len(shapes)))


@pytest.mark.timeout(600)
def test_fp64_refresh_large_4096():
    """The 4096 stress batch with the float64 statistics update: its rank-32 signal sits on
    a noise floor near 1e-6 lam_max that float32 does not resolve (the float32 run compares
    P from the GPU's own root there); in float64 the whole step is compared from the
    pre-step state where the codes agree.  Every side orthonormal, codes of a sample
    bit-exact; the first block against the oracle over the first two steps."""
    require_gpu()
    wl = get_workload("large_4096")
    shapes = wl.shapes
    announce("full size large_4096 fp64: oracle on block 0, steps 1-2")
    w = _run_teacher_forced(shapes, wl.gradients, 2, beta=wl.beta, eps=wl.eps, k=wl.bjorck_iters,
                            power_iters=wl.power_iters, root_interval=wl.root_interval, root_cache=True,
                            label="large_4096 fp64", qr="auto", sample=[0], use_step=True, fp64=True,
                            all_sides=_side_checks(shapes, 4, seed=len(shapes)))
    assert w["stat"] <= 1e-12, w
