"""Coupled Newton inverse 4th root on the MFMA GEMM against the oracle ("Shampoo --
Second-Order Optimizer", section "Computing the inverse fourth root", matrix-multiply
route), batched over matrices of several orders.  The GPU runs the iteration in float32:
after the same number of iterations its X must match the oracle's float64 iterate within
a relative Frobenius error of 1e-3, and at convergence the float64 inverse root by
eigendecomposition within the same bound (measured: at most 6.3e-6, on the order-1024 EMA
factor; each iteration is four float32 products whose rounding the next iterations
partly correct)."""

import numpy as np
import pytest
import torch

from oracle import ablation as ab
from oracle import newton as nw
from tests.gpu_util import announce, rel_fro, require_gpu, to_dev
from workloads import get_workload

pytestmark = pytest.mark.gpu

TOL = 1e-3


def _factors():
    rng = np.random.default_rng(7)
    out = []
    for p in (1, 5, 64, 130):
        B = rng.standard_normal((p, p + 3))
        out.append(B @ B.T / (p + 3))
    wl = get_workload("single_1024")
    out.append(ab.ema_factor([wl.block_gradient(0, t) for t in range(1, 11)], wl.beta))
    return out


@pytest.mark.parametrize("iters", [6, 25])
def test_newton_matches_oracle(iters):
    require_gpu()
    from bit_quantized_shampoo_amd import inverse_root
    Ls = _factors()
    eps = 1e-3
    announce(f"newton inverse root iters={iters} orders={[L.shape[0] for L in Ls]}")
    Xs, _ = inverse_root([to_dev(L.astype(np.float32)) for L in Ls], eps=eps, iters=iters)
    torch.cuda.synchronize()
    for L, X in zip(Ls, Xs):
        # the oracle from the same float32 input
        ref = nw.coupled_newton_inverse_root(L.astype(np.float32).astype(np.float64), eps, iters)
        e = rel_fro(X.cpu().numpy(), ref)
        announce(f"  order {L.shape[0]}: {e:.3e} against the oracle's iterate")
        assert e <= TOL, (L.shape, iters, e)
        if iters == 25:
            truth = ab.inverse_root(L.astype(np.float32).astype(np.float64), eps)
            e2 = rel_fro(X.cpu().numpy(), truth)
            announce(f"  order {L.shape[0]}: {e2:.3e} against the eigendecomposition")
            assert e2 <= TOL, (L.shape, "vs eigendecomposition", e2)


def test_newton_zero_iterations_and_bad_args():
    require_gpu()
    from bit_quantized_shampoo_amd import inverse_root
    from bit_quantized_shampoo_amd._lib import Shampoo4Error
    announce("newton edge cases")
    A = to_dev(np.diag([4.0, 16.0]).astype(np.float32))
    (X,), _ = inverse_root([A], eps=0.0, iters=0)       # X = c^(-1/4) I
    torch.cuda.synchronize()
    c = np.sqrt(4.0 ** 2 + 16.0 ** 2)
    assert np.allclose(X.cpu().numpy(), c ** -0.25 * np.eye(2), rtol=1e-6)
    with pytest.raises(Shampoo4Error):
        inverse_root([A], eps=-1.0)
    with pytest.raises(ValueError):
        inverse_root([to_dev(np.zeros((2, 3), np.float32))])
