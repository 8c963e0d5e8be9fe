"""Host-only checks of libshampoo4.so: it loads, exports every symbol the header
declares, its codebook equals the oracle's bit for bit, and host-side planning /
validation behave as documented.  No device call is made."""

import ctypes
import os
import re

import numpy as np
import pytest

from bit_quantized_shampoo_amd import _lib as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "shampoo4.h")


def _lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("library not built (run __graft_entry__.build())")
    return L.lib()


def declared_symbols():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"SHAMPOO4_API[^;(]*?\b(shampoo4_\w+)\s*\(", text)))


def test_header_declares_the_binding_surface():
    assert declared_symbols() == sorted(L.EXPORTED)


def test_library_exports_every_declared_symbol():
    lib = _lib()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    assert lib.shampoo4_abi_version() == 1


@pytest.mark.parametrize("name", ["ls", "dt"])
def test_codebook_matches_oracle_bitwise(name):
    _lib()
    from bit_quantized_shampoo_amd.shampoo4 import codebook
    from oracle import codec
    lv, mp = codebook(name)
    assert np.array_equal(np.array(lv, np.float32).view(np.uint32), codec.levels(name).view(np.uint32))
    assert np.array_equal(np.array(mp, np.float32).view(np.uint32), codec.midpoints(name).view(np.uint32))


def test_unknown_codebook_rejected():
    lib = _lib()
    lv = (ctypes.c_float * 16)()
    mp = (ctypes.c_float * 15)()
    assert lib.shampoo4_codebook_ex(2, lv, mp) == L.EINVAL
    assert lib.shampoo4_quantize_ex(None, 5, 64, 7, None, None, None) == L.EINVAL
    assert lib.shampoo4_dequantize_ex(None, None, 5, 64, -1, None, None) == L.EINVAL
    assert lib.shampoo4_dequantize_ex(None, None, 0, 64, L.CODEBOOK_DYNAMIC_TREE, None, None) == L.OK


def _plan(shapes, **kw):
    lib = _lib()
    cfg = L.Config(kw.get("beta", 0.95), kw.get("eps", 1e-6), kw.get("qblock", 64),
                   kw.get("k", 1), kw.get("pi", 1), kw.get("flags", 0))
    arr = (L.Shape * len(shapes))(*[L.Shape(m, n) for m, n in shapes])
    sb, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    st = lib.shampoo4_plan(ctypes.byref(cfg), len(shapes), arr, ctypes.byref(sb), ctypes.byref(wb))
    return st, sb.value, wb.value


def test_plan_sizes():
    st, sb, wb = _plan([(64, 32)])
    assert st == L.OK
    # state: per side codes + scales + lam + root codes + root scales + d, 256-byte aligned pieces
    def side(p):
        nqb = (p * p + 63) // 64
        al = lambda b: (b + 255) // 256 * 256
        return 2 * al(nqb * 32) + 2 * al(nqb * 4) + 2 * al(p * 4)
    assert sb == side(64) + side(32)
    assert wb > 7 * (64 * 64 + 32 * 32) * 4
    st2, sb2, wb2 = _plan([(64, 32), (1024, 1024)])
    assert st2 == L.OK and sb2 > sb and wb2 > wb


@pytest.mark.parametrize("shapes,kw,status", [
    ([(0, 4)], {}, L.ESHAPE),
    ([(8193, 4)], {}, L.ESHAPE),
    ([(4, 4)], {"qblock": 32}, L.EINVAL),
    ([(4, 4)], {"beta": 1.5}, L.EINVAL),
    ([(4, 4)], {"eps": -1.0}, L.EINVAL),
    ([(4, 4)], {"k": -1}, L.EINVAL),
    ([(4, 4)], {"k": 17}, L.EINVAL),
    ([(4, 4)], {"pi": 0}, L.EINVAL),
    ([(4, 4)], {"flags": 1024}, L.EINVAL),
    ([(4, 4)], {"flags": L.FLAG_DEBUG}, L.OK),
    ([(4, 4)], {"flags": L.FLAG_FP32_MFMA}, L.OK),
    ([(4, 4)], {"flags": L.FLAG_FP32_MFMA | L.FLAG_FP64_REFRESH | L.FLAG_ROOT_CACHE}, L.OK),
    ([(4, 4)], {"flags": L.FLAG_FP64_REFRESH}, L.OK),
    ([(4, 4)], {"flags": L.FLAG_FP64_REFRESH | L.FLAG_QR_LOOKAHEAD}, L.EINVAL),
    ([(4, 4)], {"flags": L.FLAG_FP64_REFRESH | L.FLAG_FP32_STATE}, L.EINVAL),
    ([(4, 4)], {"flags": L.FLAG_FP64_REFRESH | L.FLAG_QR_BLOCKED | L.FLAG_DT_CODEBOOK}, L.OK),
    ([(4, 4)], {"flags": L.FLAG_DT_CODEBOOK}, L.OK),
    ([(4, 4)], {"flags": L.FLAG_DT_CODEBOOK | L.FLAG_FP32_STATE}, L.EINVAL),
    ([(4, 4)], {"flags": L.FLAG_GRAPHS}, L.OK),
    ([(4, 4)], {"flags": L.FLAG_FP32_STATE}, L.OK),
    ([(4, 4)], {"flags": L.FLAG_QR_BLOCKED | L.FLAG_QR_LOOKAHEAD}, L.EINVAL),
    ([(4, 4)], {"flags": L.FLAG_QR_BLOCKED}, L.OK),
    ([(4, 4)], {"flags": L.FLAG_QR_LOOKAHEAD}, L.OK),
    ([(1, 1)], {}, L.OK),
    ([(8192, 1)], {}, L.OK),
])
def test_plan_validation(shapes, kw, status):
    st, _, _ = _plan(shapes, **kw)
    assert st == status


def test_strerror_and_gemm_workspace():
    lib = _lib()
    for s in range(7):
        assert isinstance(lib.shampoo4_strerror(s), bytes)
    assert lib.shampoo4_gemm_workspace_bytes(3) >= 3 * 128 + 16


def test_null_arguments_rejected_on_host():
    lib = _lib()
    assert lib.shampoo4_update_stats(None, None, None) == L.EINVAL
    assert lib.shampoo4_refresh_root(None, None) == L.EINVAL
    assert lib.shampoo4_precondition(None, None, None) == L.EINVAL
    assert lib.shampoo4_step(None, None, 0, None) == L.EINVAL
    assert lib.shampoo4_step(None, None, 1, None) == L.EINVAL
    assert lib.shampoo4_destroy(None) == L.EINVAL
    assert lib.shampoo4_quantize(None, 5, 64, None, None, None) == L.EINVAL
    assert lib.shampoo4_quantize(None, 5, 32, None, None, None) == L.EINVAL
    assert lib.shampoo4_dequantize(None, None, 0, 64, None, None) == L.OK


def test_inverse_root_workspace_sizes():
    lib = _lib()
    i32 = ctypes.c_int32
    p = (i32 * 3)(1024, 77, 1)
    need = lib.shampoo4_inverse_root_workspace_bytes(3, p)
    assert need >= 7 * 4 * (1024 * 1024 + 77 * 77 + 1)
    bad = (i32 * 1)(0)
    assert lib.shampoo4_inverse_root_workspace_bytes(1, bad) == 0
    assert lib.shampoo4_inverse_root(1, bad, None, None, 0.0, 1, None, None, None, 0, None) == L.EINVAL


def test_shape_limits_by_side_kind():
    """A diagonal side may reach 65536, a side with eigenvectors 8192; unknown side bits
    are rejected (host-only planning)."""
    _lib()
    from bit_quantized_shampoo_amd import Shampoo4Config
    from bit_quantized_shampoo_amd.shampoo4 import plan
    sb, wb = plan([(16, 65536)], Shampoo4Config(), diagonal=[(False, True)])
    assert sb > 0 and wb > 0
    with pytest.raises(L.Shampoo4Error) as e:
        plan([(16, 65537)], Shampoo4Config(), diagonal=[(False, True)])
    assert e.value.status == L.ESHAPE
    with pytest.raises(L.Shampoo4Error) as e:
        plan([(16, 9000)], Shampoo4Config(), diagonal=[(True, False)])
    assert e.value.status == L.ESHAPE
    cfg = L.Config(0.95, 1e-6, 64, 1, 1, 0)
    arr = (L.Shape * 1)(L.Shape(8, 8))
    bad = (ctypes.c_uint8 * 1)(4)
    s0, s1 = ctypes.c_size_t(0), ctypes.c_size_t(0)
    assert L.lib().shampoo4_plan_ex(ctypes.byref(cfg), 1, arr, bad, ctypes.byref(s0), ctypes.byref(s1)) == L.EINVAL


def test_diagonal_sides_hold_no_eigenvectors():
    """A diagonal side's state is its statistic and d only, and its workspace holds no p x p
    matrices: the both-diagonal plan of a block is far smaller than the full one."""
    _lib()
    from bit_quantized_shampoo_amd import Shampoo4Config
    from bit_quantized_shampoo_amd.shampoo4 import plan
    sb_full, wb_full = plan([(512, 512)], Shampoo4Config())
    sb_diag, wb_diag = plan([(512, 512)], Shampoo4Config(), diagonal=[(True, True)])
    # per side: four empty 256-byte-aligned pieces (codes, scales, root codes, root scales), lam, d
    assert sb_diag == 2 * (4 * 256 + 2 * 512 * 4)
    assert wb_diag < wb_full // 4
