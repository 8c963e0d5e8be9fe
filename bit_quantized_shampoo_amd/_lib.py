"""ctypes view of libshampoo4.so (the C ABI declared in include/shampoo4.h).

Argument marshalling only: every step of the method runs in the library's
HIP kernels.  Loading fails loudly when the library has not been built.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libshampoo4.so")

OK, EINVAL, ESHAPE, EALIGN, ESMALLBUF, EHIP, ENONFINITE = range(7)
FLAG_ROOT_CACHE = 1
FLAG_KEEP_STATE = 2
FLAG_QR_BLOCKED = 4
FLAG_QR_LOOKAHEAD = 8
FLAG_FP32_STATE = 16
FLAG_GRAPHS = 32
FLAG_DT_CODEBOOK = 64
FLAG_FP64_REFRESH = 128
FLAG_FP32_MFMA = 256
FLAG_DEBUG = 512
DIAG_L = 1
DIAG_R = 2
CODEBOOK_LINEAR_SQUARE = 0
CODEBOOK_DYNAMIC_TREE = 1

BUF_CODES, BUF_SCALES, BUF_EIG, BUF_ROOT_CODES, BUF_ROOT_SCALES, BUF_ROOT_D = range(6)
BUF_V, BUF_STAT, BUF_Q, BUF_ROOT_V, BUF_ROOT_MAT, BUF_STAT64, BUF_Q64 = 16, 17, 18, 19, 20, 21, 22

EXPORTED = [
    "shampoo4_abi_version", "shampoo4_strerror", "shampoo4_plan", "shampoo4_init",
    "shampoo4_update_stats", "shampoo4_refresh_root", "shampoo4_precondition", "shampoo4_step",
    "shampoo4_check", "shampoo4_destroy", "shampoo4_layout", "shampoo4_quantize",
    "shampoo4_dequantize", "shampoo4_codebook", "shampoo4_quantize_ex", "shampoo4_dequantize_ex",
    "shampoo4_codebook_ex", "shampoo4_gemm_workspace_bytes",
    "shampoo4_gemm_batched", "shampoo4_timing", "shampoo4_timing_report", "shampoo4_graft",
    "shampoo4_inverse_root_workspace_bytes", "shampoo4_inverse_root", "shampoo4_plan_ex", "shampoo4_init_ex",
    "shampoo4_gemm_batched_static", "shampoo4_gemm_batched_ex",
]

GRAFT_SGD, GRAFT_ADAM = 0, 1
GEMM_AUTO, GEMM_FP32, GEMM_X3 = 0, 1, 2
GEMM_STATIC_MAX = 2048


class Config(ctypes.Structure):
    _fields_ = [("beta", ctypes.c_float), ("eps", ctypes.c_float), ("qblock", ctypes.c_int32),
                ("bjorck_iters", ctypes.c_int32), ("power_iters", ctypes.c_int32),
                ("flags", ctypes.c_uint32)]


class Shape(ctypes.Structure):
    _fields_ = [("m", ctypes.c_int32), ("n", ctypes.c_int32)]


class Io(ctypes.Structure):
    _fields_ = [("G", ctypes.c_void_p), ("ldg", ctypes.c_int64),
                ("P", ctypes.c_void_p), ("ldp", ctypes.c_int64)]


class GraftConfig(ctypes.Structure):
    _fields_ = [("mode", ctypes.c_int32), ("step", ctypes.c_int32), ("lr", ctypes.c_float),
                ("eps_graft", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps_adam", ctypes.c_float)]


class GraftIo(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("ldw", ctypes.c_int64), ("M", ctypes.c_void_p),
                ("V", ctypes.c_void_p)]


class Shampoo4Error(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {strerror(status)} (status {status})")


_lib = None


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python -m bit_quantized_shampoo_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    vp, i32, i64, u32, sz, f32 = (ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_uint32,
                                  ctypes.c_size_t, ctypes.c_float)
    st = ctypes.c_int
    sig = {
        "shampoo4_abi_version": (i32, []),
        "shampoo4_strerror": (ctypes.c_char_p, [st]),
        "shampoo4_plan": (st, [ctypes.POINTER(Config), i32, ctypes.POINTER(Shape),
                               ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "shampoo4_init": (st, [ctypes.POINTER(Config), i32, ctypes.POINTER(Shape), vp, sz, vp, sz, vp,
                               ctypes.POINTER(vp)]),
        "shampoo4_plan_ex": (st, [ctypes.POINTER(Config), i32, ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_uint8),
                                  ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "shampoo4_init_ex": (st, [ctypes.POINTER(Config), i32, ctypes.POINTER(Shape), ctypes.POINTER(ctypes.c_uint8),
                                  vp, sz, vp, sz, vp, ctypes.POINTER(vp)]),
        "shampoo4_update_stats": (st, [vp, ctypes.POINTER(Io), vp]),
        "shampoo4_refresh_root": (st, [vp, vp]),
        "shampoo4_precondition": (st, [vp, ctypes.POINTER(Io), vp]),
        "shampoo4_step": (st, [vp, ctypes.POINTER(Io), i32, vp]),
        "shampoo4_check": (st, [vp, vp, ctypes.POINTER(u32)]),
        "shampoo4_destroy": (st, [vp]),
        "shampoo4_layout": (st, [vp, i32, i32, ctypes.c_int, ctypes.POINTER(sz), ctypes.POINTER(sz)]),
        "shampoo4_quantize": (st, [vp, i64, i32, vp, vp, vp]),
        "shampoo4_dequantize": (st, [vp, vp, i64, i32, vp, vp]),
        "shampoo4_codebook": (st, [ctypes.POINTER(f32), ctypes.POINTER(f32)]),
        "shampoo4_quantize_ex": (st, [vp, i64, i32, i32, vp, vp, vp]),
        "shampoo4_dequantize_ex": (st, [vp, vp, i64, i32, i32, vp, vp]),
        "shampoo4_codebook_ex": (st, [i32, ctypes.POINTER(f32), ctypes.POINTER(f32)]),
        "shampoo4_gemm_workspace_bytes": (sz, [i32]),
        "shampoo4_gemm_batched": (st, [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                       ctypes.POINTER(i32), f32, ctypes.POINTER(vp), ctypes.POINTER(i64),
                                       ctypes.POINTER(vp), ctypes.POINTER(i64), f32, ctypes.POINTER(vp),
                                       ctypes.POINTER(i64), ctypes.POINTER(vp), ctypes.POINTER(i64),
                                       vp, sz, vp]),
        "shampoo4_gemm_batched_ex": (st, [i32, i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                          ctypes.POINTER(i32), f32, ctypes.POINTER(vp), ctypes.POINTER(i64),
                                          ctypes.POINTER(vp), ctypes.POINTER(i64), f32, ctypes.POINTER(vp),
                                          ctypes.POINTER(i64), ctypes.POINTER(vp), ctypes.POINTER(i64),
                                          vp, sz, vp]),
        "shampoo4_gemm_batched_static": (st, [i32, i32, i32, ctypes.POINTER(i32), ctypes.POINTER(i32),
                                              ctypes.POINTER(i32), f32, ctypes.POINTER(vp), ctypes.POINTER(i64),
                                              ctypes.POINTER(vp), ctypes.POINTER(i64), f32, ctypes.POINTER(vp),
                                              ctypes.POINTER(i64), ctypes.POINTER(vp), ctypes.POINTER(i64), vp]),
        "shampoo4_timing": (st, [vp, i32]),
        "shampoo4_inverse_root_workspace_bytes": (sz, [i32, ctypes.POINTER(i32)]),
        "shampoo4_inverse_root": (st, [i32, ctypes.POINTER(i32), ctypes.POINTER(vp), ctypes.POINTER(i64), f32, i32,
                                       ctypes.POINTER(vp), ctypes.POINTER(i64), vp, sz, vp]),
        "shampoo4_graft": (st, [vp, ctypes.POINTER(Io), ctypes.POINTER(GraftIo), ctypes.POINTER(GraftConfig), vp]),
        "shampoo4_timing_report": (st, [vp, ctypes.POINTER(i32), ctypes.POINTER(ctypes.c_char_p),
                                        ctypes.POINTER(i64), ctypes.POINTER(ctypes.c_double),
                                        ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_double)]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(L, name)
        fn.restype = res
        fn.argtypes = args
    _lib = L
    return L


def strerror(status: int) -> str:
    try:
        return lib().shampoo4_strerror(status).decode()
    except ImportError:
        return f"status {status}"


def check(status: int, what: str):
    if status != OK:
        raise Shampoo4Error(status, what)
