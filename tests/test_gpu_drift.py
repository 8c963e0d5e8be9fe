"""Free-running drift of the GPU trajectory from the oracle's (a diagnostic: not a parity
gate).

The 1024 block workload (one [1024, 1024] block of anisotropic gradients, statistics every
step, root refresh every 10 steps, 100 steps) runs free: the GPU through shampoo4_step
with cached roots (the benchmark's path) and the oracle from the same gradients, each
from its own state, never forced to agree.  Reported per step: the relative Frobenius
gap of the preconditioned gradients P; at every 10th step the share of 4-bit codes of U
and of the root snapshot that differ between the two states (both sides), and the
relative gap of the eigenvalues.  Beside them, the GPU's 4-bit trajectory against the
GPU's 32-bit one (U kept in float32, the baseline the abstract of "4-bit Shampoo for
Memory-Efficient Network Training" compares with): the method's own 4-bit effect.

Nothing here fixes how far free trajectories may drift (small float32 differences are
amplified by each refresh's choice of eigenvectors within near-degenerate eigenspaces);
asserted are only what holds at any drift: every P finite, the same non-zero pattern of
work (P non-zero), and the gaps printed for the record.
"""

import numpy as np
import pytest
import torch

from oracle import shampoo4 as o
from tests.gpu_util import announce, rel_fro, require_gpu, to_dev
from workloads import get_workload

pytestmark = pytest.mark.gpu


def _lo_hi(codes):
    c = np.asarray(codes, np.uint8)
    return np.concatenate([c & 15, c >> 4])


def test_single_1024_free_running_drift():
    require_gpu()
    from bit_quantized_shampoo_amd import Shampoo4Blocks, Shampoo4Config
    wl = get_workload("single_1024")
    steps, T = wl.steps, wl.root_interval
    cfg = dict(beta=wl.beta, eps=wl.eps, bjorck_iters=wl.bjorck_iters, root_cache=True)
    announce(f"drift single_1024: {steps} steps, root every {T}")
    gpu = Shampoo4Blocks(wl.shapes, Shampoo4Config(**cfg))
    gpu32 = Shampoo4Blocks(wl.shapes, Shampoo4Config(fp32_state=True, **cfg))
    orc = o.Shampoo4Oracle(wl.shapes, beta=wl.beta, eps=wl.eps, bjorck_iters=wl.bjorck_iters)
    rows = []
    for t in range(1, steps + 1):
        Gs = wl.gradients(t)
        Gd = [to_dev(G) for G in Gs]
        P = gpu.step(Gd, t, T)[0]
        P32 = gpu32.step(Gd, t, T)[0]
        torch.cuda.synchronize()
        Pg = P.cpu().numpy()
        P32g = P32.cpu().numpy()
        Po = orc.step(Gs, t, T)[0]
        assert np.all(np.isfinite(Pg)) and np.all(np.isfinite(P32g))
        assert np.linalg.norm(Pg) > 0
        row = {"t": t, "P_vs_oracle": rel_fro(Pg, Po), "P4_vs_P32": rel_fro(Pg, P32g),
               "P32_vs_oracle": rel_fro(P32g, Po)}
        if t % T == 0:
            flips, roots, total = 0, 0, 0
            lam_gap = []
            for s in (0, 1):
                st = gpu.side_state(0, s)
                os_ = orc.sides[0][s]
                a, b = _lo_hi(st["codes"]), _lo_hi(os_.codes)
                flips += int(np.count_nonzero(a != b))
                roots += int(np.count_nonzero(_lo_hi(st["root_codes"]) != _lo_hi(os_.root_codes)))
                total += a.size
                lam_gap.append(rel_fro(st["lam"], os_.lam))
            row.update(code_flips=flips / total, root_code_flips=roots / total, lam_gap=max(lam_gap))
        rows.append(row)
        if t % T == 0 or t <= 3:
            print("[drift] " + " ".join(f"{k}={v:.3e}" if isinstance(v, float) else f"{k}={v}"
                                       for k, v in row.items()), flush=True)
    gpu.close()
    gpu32.close()
    worst = max(r["P_vs_oracle"] for r in rows)
    mean = float(np.mean([r["P_vs_oracle"] for r in rows]))
    eff = float(np.mean([r["P4_vs_P32"] for r in rows]))
    print(f"[drift] summary: P vs oracle worst {worst:.3e} mean {mean:.3e}; "
          f"4-bit vs 32-bit GPU P mean {eff:.3e}", flush=True)
