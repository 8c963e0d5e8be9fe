"""The matrix-product kernels in isolation against float64 NumPy products: the fp32
matrix-core kernel (every tile shape, chosen by batch size), the three-piece bf16 kernel
on its small-batch 64 x 64 tile (auto) and forced onto 128 x 128 tiles whatever the
batch (x3), every transpose mode, ragged edges, strided and unaligned operands,
alpha/beta.  All must meet the fp32 bound 4 eps |A||B| sqrt(K + 1) elementwise; the two
three-piece tiles must agree bit for bit (each output sums the same terms in the same
order)."""

import numpy as np
import pytest
import torch

from tests.gpu_util import announce, require_gpu, to_dev

pytestmark = pytest.mark.gpu


def _check(As, Bs, Ds, ta, tb, alpha, beta, Cs):
    for i, (A, B, D) in enumerate(zip(As, Bs, Ds)):
        a = A.cpu().numpy().astype(np.float64)
        b = B.cpu().numpy().astype(np.float64)
        a = a.T if ta else a
        b = b.T if tb else b
        ref = alpha * (a @ b)
        if beta != 0.0:
            ref = ref + beta * Cs[i].cpu().numpy().astype(np.float64)
        got = D.cpu().numpy().astype(np.float64)
        # fp32 accumulation: bound by K * eps * |A||B| elementwise
        bound = 4 * np.float32(np.finfo(np.float32).eps) * (np.abs(a) @ np.abs(b)) * max(1.0, abs(alpha)) \
            * np.sqrt(a.shape[1] + 1) + 1e-30
        if beta != 0.0:
            bound = bound + 4 * np.finfo(np.float32).eps * np.abs(beta * Cs[i].cpu().numpy())
        err = np.abs(got - ref)
        assert np.all(err <= bound), (i, float(np.max(err / bound)))


@pytest.mark.parametrize("kernel", ["auto", "fp32", "x3"])
@pytest.mark.parametrize("ta", [False, True])
@pytest.mark.parametrize("tb", [False, True])
@pytest.mark.parametrize("shapes", [
    [(1, 1, 1)],
    [(5, 7, 3)],
    [(33, 65, 17)],
    [(64, 64, 64)],
    [(130, 70, 129), (31, 200, 5)],
    [(256, 256, 256)] * 3,
    [(1024, 1024, 1024)],                 # single large product
    [(1024, 1024, 1024)] * 2,             # two large products
    [(1024, 1024, 1024)] * 8,             # 512 tiles of 128 x 128: auto takes the bf16 split
    [(1000, 600, 77)] * 6,                # ragged edges on both sides
    [(32, 1000, 700)] * 2,                # skinny M
    [(1000, 32, 700)] * 2,                # skinny N (128 x 32 tiles)
    [(96, 20, 1024)] * 4,                 # skinny N, short M, long K
    [(700, 17, 33)] * 3,                  # skinny N with unaligned rows
    [(48, 60, 300)] * 3,                  # sides under 64 (64 x 64 tiles)
])
def test_gemm_modes(kernel, ta, tb, shapes):
    require_gpu()
    from bit_quantized_shampoo_amd import gemm_batched
    rng = np.random.default_rng(hash((ta, tb, len(shapes), shapes[0])) % (2 ** 32))
    As, Bs = [], []
    for (M, N, K) in shapes:
        A = rng.standard_normal((K, M) if ta else (M, K)).astype(np.float32)
        B = rng.standard_normal((N, K) if tb else (K, N)).astype(np.float32)
        As.append(to_dev(A))
        Bs.append(to_dev(B))
    announce(f"gemm kernel={kernel} ta={ta} tb={tb} shapes={shapes}")
    Ds, _ = gemm_batched(As, Bs, transA=ta, transB=tb, kernel=kernel)
    torch.cuda.synchronize()
    _check(As, Bs, Ds, ta, tb, 1.0, 0.0, None)


@pytest.mark.parametrize("kernel", ["auto", "x3"])
def test_gemm_alpha_beta_and_strides(kernel):
    require_gpu()
    from bit_quantized_shampoo_amd import gemm_batched
    rng = np.random.default_rng(7)
    big = to_dev(rng.standard_normal((300, 301)).astype(np.float32))
    A = big[5:105, 3:83]          # strided view [100, 80], ld 301 (unaligned rows)
    B = to_dev(rng.standard_normal((80, 90)).astype(np.float32))
    C = to_dev(rng.standard_normal((100, 90)).astype(np.float32))
    D = torch.empty((100, 90), dtype=torch.float32, device="cuda")
    announce(f"gemm alpha/beta strided kernel={kernel}")
    gemm_batched([A], [B], [D], alpha=-0.5, beta=1.5, Cs=[C], kernel=kernel)
    torch.cuda.synchronize()
    _check([A], [B], [D], False, False, -0.5, 1.5, [C])
    # K = 0 gives beta * C
    A0 = big[5:105, 3:3]          # [100, 0] view with a valid base pointer
    B0 = B[:0, :]                 # [0, 90]
    D0 = torch.empty((100, 90), dtype=torch.float32, device="cuda")
    announce(f"gemm K=0 kernel={kernel}")
    gemm_batched([A0], [B0], [D0], alpha=1.0, beta=2.0, Cs=[C], kernel=kernel)
    torch.cuda.synchronize()
    assert torch.equal(D0, 2.0 * C)


@pytest.mark.parametrize("ta,tb", [(False, False), (True, False), (False, True), (True, True)])
@pytest.mark.parametrize("shapes", [
    [(1024, 1024, 1024)] * 2,             # the single-block products of a 1024 block
    [(130, 70, 129), (31, 200, 5)],       # ragged, K not a multiple of 16 or 32
    [(300, 260, 1000)] * 3,               # K a multiple of 8, not of 32
])
def test_x3_tiles_bit_identical(ta, tb, shapes):
    """64 x 64 tiles (32-k slices) and 128 x 128 tiles (16-k slices) of the three-piece
    kernel: every output takes the same six piece products per 16 k in the same order, so
    the results are equal bit for bit (the step's precondition beside the QR chain relies
    on it)."""
    require_gpu()
    from bit_quantized_shampoo_amd import gemm_batched
    rng = np.random.default_rng(len(shapes) * 7 + 2 * ta + tb)
    As, Bs = [], []
    for (M, N, K) in shapes:
        As.append(to_dev(rng.standard_normal((K, M) if ta else (M, K)).astype(np.float32)))
        Bs.append(to_dev(rng.standard_normal((N, K) if tb else (K, N)).astype(np.float32)))
    announce(f"x3 tiles bit-identical ta={ta} tb={tb} shapes={shapes}")
    D64, _ = gemm_batched(As, Bs, transA=ta, transB=tb, kernel="auto")
    D128, _ = gemm_batched(As, Bs, transA=ta, transB=tb, kernel="x3")
    torch.cuda.synchronize()
    _check(As, Bs, D64, ta, tb, 1.0, 0.0, None)
    for a, b in zip(D64, D128):
        assert torch.equal(a, b)
