"""The abstract's ablation on the GPU kernels ("4-bit Shampoo for Memory-Efficient Network
Training": 4-bit eigenvector matrix versus 4-bit preconditioner, the effect of rectifying
orthogonality, and linear-square versus dynamic tree codes).  The eigenvector matrix and
the factor are quantized and dequantized by the library's codec, and the Bjorck
rectification runs on its MFMA GEMM;
only the float64 eigendecompositions (truth, and the inverse root of the dequantized
factor) run on the host.  The errors must agree with the oracle's (relative 1e-3: the
GEMM rectifies in float32) and reproduce the claim."""

import numpy as np
import pytest
import torch

from oracle import ablation as ab
from tests.gpu_util import announce, require_gpu, to_dev
from workloads import get_workload

pytestmark = pytest.mark.gpu


def _gpu_bjorck(V, iters):
    from bit_quantized_shampoo_amd import gemm_batched
    for _ in range(iters):
        (W,), _ = gemm_batched([V], [V], transA=True)
        (V,), _ = gemm_batched([V], [W], alpha=-0.5, beta=1.5, Cs=[V])
    return V


@pytest.mark.parametrize("workload", ["single_64x32", "cnn_batch", "single_1024"])
def test_ablation_on_gpu_kernels(workload):
    require_gpu()
    from bit_quantized_shampoo_amd import dequantize, quantize
    wl = get_workload(workload)
    L = ab.ema_factor([wl.block_gradient(0, t) for t in range(1, 11)], wl.beta)
    p = L.shape[0]
    eps = 1e-6
    announce(f"ablation {workload} p={p}")
    truth = ab.inverse_root(L, eps)
    lam, U = ab.eigh_desc(L)
    # 4-bit eigenvectors through the GPU codec, rectified on the GPU GEMM
    c, s = quantize(to_dev(U.astype(np.float32)))
    U4 = dequantize(c, s, p * p).view(p, p)
    errs = {}
    for k, name in ((0, "eigvec4_no_rectify"), (1, "eigvec4")):
        V = _gpu_bjorck(U4.clone(), k)
        torch.cuda.synchronize()
        errs[name] = ab.rel_err(ab.root_from(V.cpu().numpy(), lam.astype(np.float32), eps), truth)
    # 4-bit preconditioner through the GPU codec
    c, s = quantize(to_dev(L.astype(np.float32)))
    L4 = dequantize(c, s, p * p).view(p, p)
    torch.cuda.synchronize()
    errs["precond4"] = ab.rel_err(ab.inverse_root(L4.cpu().numpy().astype(np.float64), eps), truth)
    # the same 4-bit eigenvectors with the dynamic tree codebook
    c, s = quantize(to_dev(U.astype(np.float32)), codebook="dt")
    V = _gpu_bjorck(dequantize(c, s, p * p, codebook="dt").view(p, p), 1)
    torch.cuda.synchronize()
    errs["eigvec4_dt"] = ab.rel_err(ab.root_from(V.cpu().numpy(), lam.astype(np.float32), eps), truth)
    ref = ab.ablation(L, eps, 1)
    announce(f"ablation {workload}: gpu {errs} oracle {ref}")
    for k, v in errs.items():
        assert abs(v - ref[k]) <= 1e-3 * ref[k], (workload, k, v, ref[k])
    assert errs["eigvec4"] < errs["precond4"]
    assert errs["eigvec4"] < errs["eigvec4_no_rectify"]
    assert errs["eigvec4"] < errs["eigvec4_dt"]       # linear-square ahead of dynamic tree
