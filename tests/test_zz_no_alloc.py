"""The allocation-free batched GEMM (shampoo4_gemm_batched_static, for callers that cannot
allocate device memory) called through the C ABI: its results equal those of
shampoo4_gemm_batched bit for bit (same kernels and descriptors, the table in the
library's static device array instead of a workspace), over two calls in a row, the
second with fewer and smaller products, and a count above the limit is refused before
anything is enqueued."""

import ctypes

import numpy as np
import pytest
import torch

from bit_quantized_shampoo_amd import _lib as L
from tests.gpu_util import announce, require_gpu

pytestmark = pytest.mark.gpu


def _args(As, Bs, Ds, Cs, transA, transB):
    n = len(As)
    i32, i64, vp = ctypes.c_int32 * n, ctypes.c_int64 * n, ctypes.c_void_p * n
    Ms, Ns, Ks = [], [], []
    for A, B in zip(As, Bs):
        M, K = (A.shape[1], A.shape[0]) if transA else (A.shape[0], A.shape[1])
        N = B.shape[0] if transB else B.shape[1]
        Ms.append(M); Ns.append(N); Ks.append(K)
    return [n, int(transA), int(transB), i32(*Ms), i32(*Ns), i32(*Ks), 1.25,
            vp(*[a.data_ptr() for a in As]), i64(*[a.stride(0) for a in As]),
            vp(*[b.data_ptr() for b in Bs]), i64(*[b.stride(0) for b in Bs]), 0.5,
            vp(*[c.data_ptr() for c in Cs]), i64(*[c.stride(0) for c in Cs]),
            vp(*[d.data_ptr() for d in Ds]), i64(*[d.stride(0) for d in Ds])]


def _case(rng, shapes, transA, transB):
    As, Bs, Cs = [], [], []
    for M, N, K in shapes:
        As.append(torch.from_numpy(rng.standard_normal((K, M) if transA else (M, K)).astype(np.float32)).cuda())
        Bs.append(torch.from_numpy(rng.standard_normal((N, K) if transB else (K, N)).astype(np.float32)).cuda())
        Cs.append(torch.from_numpy(rng.standard_normal((M, N)).astype(np.float32)).cuda())
    return As, Bs, Cs


def test_static_gemm_matches_workspace_gemm_over_two_calls():
    require_gpu()
    lib = L.lib()
    rng = np.random.default_rng(31)
    stream = torch.cuda.current_stream().cuda_stream
    cases = [
        ([(300, 257, 129), (64, 1000, 33), (1024, 1024, 1024), (5, 7, 3)] * 3, True, False),
        ([(40, 72, 96), (17, 9, 200)], False, True),        # the second call: fewer, smaller products
    ]
    for k, (shapes, ta, tb) in enumerate(cases):
        As, Bs, Cs = _case(rng, shapes, ta, tb)
        D1 = [torch.full((M, N), float("nan"), device="cuda") for M, N, _ in shapes]
        D2 = [torch.full((M, N), float("nan"), device="cuda") for M, N, _ in shapes]
        need = lib.shampoo4_gemm_workspace_bytes(len(shapes))
        ws = torch.empty(need, dtype=torch.uint8, device="cuda")
        announce(f"static gemm call {k + 1}: {len(shapes)} products")
        st = lib.shampoo4_gemm_batched(*_args(As, Bs, D1, Cs, ta, tb), ws.data_ptr(), need, stream)
        assert st == L.OK, L.strerror(st)
        st = lib.shampoo4_gemm_batched_static(*_args(As, Bs, D2, Cs, ta, tb), stream)
        assert st == L.OK, L.strerror(st)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(zip(D1, D2)):
            assert torch.equal(a, b), (k, i)
            # and the product itself
            ref = 1.25 * ((As[i].T if ta else As[i]).double() @ (Bs[i].T if tb else Bs[i]).double()) + 0.5 * Cs[i].double()
            assert float((a.double() - ref).norm() / ref.norm()) <= 1e-5, (k, i)


def test_static_gemm_refuses_more_than_its_table_holds():
    require_gpu()
    lib = L.lib()
    n = L.GEMM_STATIC_MAX + 1
    A = torch.zeros((4, 4), device="cuda")
    args = _args([A] * n, [A] * n, [A] * n, [A] * n, False, False)
    assert lib.shampoo4_gemm_batched_static(*args, torch.cuda.current_stream().cuda_stream) == L.ESMALLBUF
    # zero products: nothing to do
    assert lib.shampoo4_gemm_batched_static(0, 0, 0, None, None, None, 1.0, None, None, None, None, 0.0,
                                            None, None, None, None, None) == L.OK
