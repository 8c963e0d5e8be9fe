"""Thin PyTorch-facing binding of the C ABI (same names as include/shampoo4.h).

PyTorch provides device memory and the current stream; every computation is a
kernel of libshampoo4.so.  There is no CPU fallback: without a GPU or without
the built library these calls raise.
"""

from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from . import _lib as L


def _stream_ptr(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _ptr(t: torch.Tensor) -> int:
    return t.data_ptr()


def _require_gpu_tensor(t: torch.Tensor, dtype, what: str):
    if not isinstance(t, torch.Tensor) or not t.is_cuda:
        raise TypeError(f"{what} must be a CUDA (HIP) tensor")
    if t.dtype != dtype:
        raise TypeError(f"{what} must be {dtype}, got {t.dtype}")


def _matrix_io(G: torch.Tensor, P: torch.Tensor | None, m: int, n: int, what: str) -> L.Io:
    _require_gpu_tensor(G, torch.float32, what)
    if G.dim() != 2 or tuple(G.shape) != (m, n):
        raise ValueError(f"{what} must have shape {(m, n)}, got {tuple(G.shape)}")
    if G.stride(1) != 1 and n > 1:
        raise ValueError(f"{what} must be row-major (unit column stride)")
    io = L.Io(_ptr(G), max(G.stride(0), n) if m > 1 else n, 0, n)
    if P is not None:
        _require_gpu_tensor(P, torch.float32, "P")
        if tuple(P.shape) != (m, n) or (P.stride(1) != 1 and n > 1):
            raise ValueError(f"P must be a row-major {(m, n)} tensor")
        io.P = _ptr(P)
        io.ldp = max(P.stride(0), n) if m > 1 else n
    return io


@dataclass
class Shampoo4Config:
    beta: float = 0.95
    eps: float = 1e-6
    qblock: int = 64
    bjorck_iters: int = 1
    power_iters: int = 1
    root_cache: bool = False
    qr_schedule: str = "auto"       # "auto", "blocked" or "lookahead"
    fp32_state: bool = False        # keep U in float32 (the 32-bit baseline) instead of 4-bit codes
    graphs: bool = False            # replay update_stats from a captured HIP graph
    codebook: str = "ls"            # 4-bit codebook of U: "ls" linear-square, "dt" dynamic tree
    fp64_refresh: bool = False      # statistics update (Bjorck .. Rayleigh quotients) in float64
    fp32_mfma: bool = False         # every product on the fp32 matrix cores (no three-piece bf16 split)
    debug: bool = False             # descriptor range checks at init, NaN-filled temporaries per call

    def c(self, keep_state: bool = False) -> L.Config:
        flags = (L.FLAG_ROOT_CACHE if self.root_cache else 0) | (L.FLAG_KEEP_STATE if keep_state else 0)
        if self.qr_schedule not in ("auto", "blocked", "lookahead"):
            raise ValueError(f"qr_schedule must be auto, blocked or lookahead, not {self.qr_schedule!r}")
        flags |= {"auto": 0, "blocked": L.FLAG_QR_BLOCKED, "lookahead": L.FLAG_QR_LOOKAHEAD}[self.qr_schedule]
        if self.fp32_state:
            flags |= L.FLAG_FP32_STATE
        if self.graphs:
            flags |= L.FLAG_GRAPHS
        flags |= {"ls": 0, "dt": L.FLAG_DT_CODEBOOK}[self.codebook]
        if self.fp64_refresh:
            flags |= L.FLAG_FP64_REFRESH
        if self.fp32_mfma:
            flags |= L.FLAG_FP32_MFMA
        if self.debug:
            flags |= L.FLAG_DEBUG
        return L.Config(self.beta, self.eps, self.qblock, self.bjorck_iters, self.power_iters, flags)


def _diag_bits(diagonal, nblocks: int):
    """Per-block bytes of diagonal sides from pairs (side L diagonal, side R diagonal)."""
    if diagonal is None:
        return None
    if len(diagonal) != nblocks:
        raise ValueError(f"diagonal needs one (L, R) pair per block ({nblocks})")
    bits = [(L.DIAG_L if dl else 0) | (L.DIAG_R if dr else 0) for dl, dr in diagonal]
    return (ctypes.c_uint8 * nblocks)(*bits)


def plan(shapes, config: Shampoo4Config, diagonal=None):
    shapes = [(int(m), int(n)) for (m, n) in shapes]
    arr = (L.Shape * len(shapes))(*[L.Shape(m, n) for (m, n) in shapes])
    sb, wb = ctypes.c_size_t(0), ctypes.c_size_t(0)
    cfg = config.c()
    L.check(L.lib().shampoo4_plan_ex(ctypes.byref(cfg), len(shapes), arr, _diag_bits(diagonal, len(shapes)),
                                     ctypes.byref(sb), ctypes.byref(wb)), "shampoo4_plan_ex")
    return sb.value, wb.value


class Shampoo4Blocks:
    """4-bit Shampoo state for a list of blocks G_b:[m_b, n_b] on one GPU.

    `diagonal`: optional per-block pairs (side L diagonal, side R diagonal) for the
    one-sided fallback of a side over the size threshold (see blocking.plan_blocks)."""

    def __init__(self, shapes, config: Shampoo4Config | None = None, device="cuda",
                 state: torch.Tensor | None = None, diagonal=None):
        self.config = config or Shampoo4Config()
        self.shapes = [(int(m), int(n)) for (m, n) in shapes]
        self.nblocks = len(self.shapes)
        self.device = torch.device(device)
        self.diagonal = [(bool(a), bool(b)) for a, b in diagonal] if diagonal is not None else None
        self._diag_arr = _diag_bits(self.diagonal, self.nblocks)
        sb, wb = plan(self.shapes, self.config, self.diagonal)
        keep = state is not None
        if keep:
            _require_gpu_tensor(state, torch.uint8, "state")
            if state.numel() != sb:
                raise ValueError(f"state must hold {sb} bytes")
            self.state = state.contiguous()
        else:
            self.state = torch.empty(sb, dtype=torch.uint8, device=self.device)
        self.workspace = torch.empty(wb, dtype=torch.uint8, device=self.device)
        self._shape_arr = (L.Shape * self.nblocks)(*[L.Shape(m, n) for (m, n) in self.shapes])
        self._ctx = ctypes.c_void_p(0)
        cfg = self.config.c(keep_state=keep)
        L.check(L.lib().shampoo4_init_ex(ctypes.byref(cfg), self.nblocks, self._shape_arr, self._diag_arr,
                                         _ptr(self.state), sb, _ptr(self.workspace), wb,
                                         _stream_ptr(), ctypes.byref(self._ctx)), "shampoo4_init_ex")

    def close(self):
        if self._ctx and self._ctx.value:
            L.lib().shampoo4_destroy(self._ctx)
            self._ctx = ctypes.c_void_p(0)

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def _io(self, grads, outs=None):
        if len(grads) != self.nblocks:
            raise ValueError(f"expected {self.nblocks} gradients, got {len(grads)}")
        ios = []
        for b, (m, n) in enumerate(self.shapes):
            ios.append(_matrix_io(grads[b], None if outs is None else outs[b], m, n, f"G[{b}]"))
        return (L.Io * self.nblocks)(*ios)

    def update_stats(self, grads, stream=None):
        io = self._io(grads)
        L.check(L.lib().shampoo4_update_stats(self._ctx, io, _stream_ptr(stream)), "shampoo4_update_stats")

    def refresh_root(self, stream=None):
        L.check(L.lib().shampoo4_refresh_root(self._ctx, _stream_ptr(stream)), "shampoo4_refresh_root")

    def precondition(self, grads, outs=None, stream=None):
        if outs is None:
            outs = [torch.empty((m, n), dtype=torch.float32, device=self.device) for (m, n) in self.shapes]
        io = self._io(grads, outs)
        L.check(L.lib().shampoo4_precondition(self._ctx, io, _stream_ptr(stream)), "shampoo4_precondition")
        return outs

    def step(self, grads, t: int, root_interval: int = 1, outs=None, stream=None):
        """update_stats, refresh_root when t % root_interval == 0, precondition, as one
        call (shampoo4_step: without a refresh, the precondition runs beside the
        statistics update on a second stream)."""
        if outs is None:
            outs = [torch.empty((m, n), dtype=torch.float32, device=self.device) for (m, n) in self.shapes]
        io = self._io(grads, outs)
        refresh = int(t % root_interval == 0)
        L.check(L.lib().shampoo4_step(self._ctx, io, refresh, _stream_ptr(stream)), "shampoo4_step")
        return outs

    def graft(self, grads, directions, weights, moments=None, *, mode: str = "sgd", lr: float = 1.0,
              eps_graft: float = 1e-8, step: int = 1, beta1: float = 0.9, beta2: float = 0.999,
              eps_adam: float = 1e-8, stream=None):
        """Grafted weight update W <- W - lr ||d_graft|| / (||P|| + eps_graft) P per block, in
        place on `weights`; `directions` are the preconditioned P.  mode "adam" needs
        `moments` = [(M, V), ...] (contiguous fp32, updated in place)."""
        if mode not in ("sgd", "adam"):
            raise ValueError(f"mode must be sgd or adam, not {mode!r}")
        adam = mode == "adam"
        if adam and moments is None:
            raise ValueError("mode adam needs moments=[(M, V), ...]")
        io = self._io(grads, directions)
        gio = (L.GraftIo * len(self.shapes))()
        for b, (m, n) in enumerate(self.shapes):
            W = weights[b]
            _require_gpu_tensor(W, torch.float32, "W")
            if tuple(W.shape) != (m, n) or (W.stride(1) != 1 and n > 1):
                raise ValueError(f"W must be a row-major {(m, n)} tensor")
            gio[b].W = _ptr(W)
            gio[b].ldw = max(W.stride(0), n) if m > 1 else n
            if adam:
                Mt, Vt = moments[b]
                for t_, nm in ((Mt, "M"), (Vt, "V")):
                    _require_gpu_tensor(t_, torch.float32, nm)
                    if tuple(t_.shape) != (m, n) or not t_.is_contiguous():
                        raise ValueError(f"{nm} must be a contiguous {(m, n)} tensor")
                gio[b].M = _ptr(Mt)
                gio[b].V = _ptr(Vt)
        cfg = L.GraftConfig(L.GRAFT_ADAM if adam else L.GRAFT_SGD, int(step), float(lr), float(eps_graft),
                            float(beta1), float(beta2), float(eps_adam))
        L.check(L.lib().shampoo4_graft(self._ctx, io, gio, ctypes.byref(cfg), _stream_ptr(stream)),
                "shampoo4_graft")
        return weights

    def check(self, stream=None) -> int:
        flags = ctypes.c_uint32(0)
        st = L.lib().shampoo4_check(self._ctx, _stream_ptr(stream), ctypes.byref(flags))
        if st not in (L.OK, L.ENONFINITE):
            L.check(st, "shampoo4_check")
        return flags.value

    # -- views for tests and checkpoints ---------------------------------------------
    def _layout(self, block: int, side: int, which: int):
        off, nbytes = ctypes.c_size_t(0), ctypes.c_size_t(0)
        L.check(L.lib().shampoo4_layout(self._ctx, block, side, which, ctypes.byref(off), ctypes.byref(nbytes)),
                "shampoo4_layout")
        return off.value, nbytes.value

    def view(self, block: int, side: int, which: int) -> torch.Tensor:
        off, nbytes = self._layout(block, side, which)
        base = self.state if which < 16 else self.workspace
        raw = base[off:off + nbytes]
        if which in (L.BUF_CODES, L.BUF_ROOT_CODES):
            return raw
        if which in (L.BUF_STAT64, L.BUF_Q64):
            p = self.shapes[block][side]
            return raw.view(torch.float64).view(p, p)
        t = raw.view(torch.float32)
        if which >= 16:
            p = self.shapes[block][side]
            return t.view(p, p)
        return t

    def eigenvectors(self, block: int, side: int, root: bool = False) -> torch.Tensor:
        """The float32 U of a side (only with fp32_state), p x p, a view into the state."""
        if not self.config.fp32_state:
            raise ValueError("eigenvectors() needs fp32_state; 4-bit states hold codes")
        p = self.shapes[block][side]
        raw = self.view(block, side, L.BUF_ROOT_CODES if root else L.BUF_CODES)
        return raw.view(torch.float32).view(p, p)

    def side_state(self, block: int, side: int) -> dict:
        """Host copies of one side's state (codes, scales, lam, root codes/scales, d)."""
        names = {"codes": L.BUF_CODES, "scales": L.BUF_SCALES, "lam": L.BUF_EIG,
                 "root_codes": L.BUF_ROOT_CODES, "root_scales": L.BUF_ROOT_SCALES, "d": L.BUF_ROOT_D}
        return {k: self.view(block, side, w).cpu().numpy().copy() for k, w in names.items()}

    def load_side_state(self, block: int, side: int, st: dict):
        names = {"codes": L.BUF_CODES, "scales": L.BUF_SCALES, "lam": L.BUF_EIG,
                 "root_codes": L.BUF_ROOT_CODES, "root_scales": L.BUF_ROOT_SCALES, "d": L.BUF_ROOT_D}
        for k, w in names.items():
            v = self.view(block, side, w)
            v.copy_(torch.as_tensor(st[k]).to(v.dtype).reshape(v.shape))

    # -- timing ------------------------------------------------------------------------
    def timing(self, enable: bool):
        L.check(L.lib().shampoo4_timing(self._ctx, 1 if enable else 0), "shampoo4_timing")

    def timing_report(self) -> dict:
        n = 32
        cnt = ctypes.c_int32(n)
        names = (ctypes.c_char_p * n)()
        launches = (ctypes.c_int64 * n)()
        ms = (ctypes.c_double * n)()
        fl = (ctypes.c_double * n)()
        by = (ctypes.c_double * n)()
        L.check(L.lib().shampoo4_timing_report(self._ctx, ctypes.byref(cnt), names, launches, ms, fl, by),
                "shampoo4_timing_report")
        return {names[i].decode(): {"launches": launches[i], "ms": ms[i], "flops": fl[i], "bytes": by[i]}
                for i in range(cnt.value)}


# -- codec and GEMM in isolation -------------------------------------------------------

def _codebook_id(codebook: str) -> int:
    return {"ls": L.CODEBOOK_LINEAR_SQUARE, "dt": L.CODEBOOK_DYNAMIC_TREE}[codebook]


def quantize(x: torch.Tensor, qblock: int = 64, stream=None, codebook: str = "ls"):
    _require_gpu_tensor(x, torch.float32, "x")
    x = x.contiguous().view(-1)
    n = x.numel()
    nqb = (n + qblock - 1) // qblock
    codes = torch.empty(nqb * qblock // 2, dtype=torch.uint8, device=x.device)
    scales = torch.empty(nqb, dtype=torch.float32, device=x.device)
    L.check(L.lib().shampoo4_quantize_ex(_ptr(x), n, qblock, _codebook_id(codebook), _ptr(codes), _ptr(scales),
                                         _stream_ptr(stream)), "shampoo4_quantize_ex")
    return codes, scales


def dequantize(codes: torch.Tensor, scales: torch.Tensor, n: int, qblock: int = 64, stream=None,
               codebook: str = "ls"):
    _require_gpu_tensor(codes, torch.uint8, "codes")
    _require_gpu_tensor(scales, torch.float32, "scales")
    x = torch.empty(n, dtype=torch.float32, device=codes.device)
    L.check(L.lib().shampoo4_dequantize_ex(_ptr(codes.contiguous()), _ptr(scales.contiguous()), n, qblock,
                                           _codebook_id(codebook), _ptr(x), _stream_ptr(stream)),
            "shampoo4_dequantize_ex")
    return x


def codebook(name: str = "ls"):
    lv = (ctypes.c_float * 16)()
    mp = (ctypes.c_float * 15)()
    L.check(L.lib().shampoo4_codebook_ex(_codebook_id(name), lv, mp), "shampoo4_codebook_ex")
    return list(lv), list(mp)


def gemm_batched(As, Bs, Ds=None, transA=False, transB=False, alpha=1.0, beta=0.0, Cs=None,
                 workspace: torch.Tensor | None = None, stream=None, kernel: str = "auto"):
    """D_i = alpha op(A_i) op(B_i) + beta C_i on the MFMA kernels (row-major 2-D tensors).
    kernel: "auto" (tile shape by batch; 128 x 128 and 64 x 64 launches on the three-piece bf16 kernel),
    "fp32" (fp32 matrix cores only) or "x3" (128 x 128 tiles on the three-piece bf16 kernel
    whatever the batch)."""
    kinds = {"auto": L.GEMM_AUTO, "fp32": L.GEMM_FP32, "x3": L.GEMM_X3}
    if kernel not in kinds:
        raise ValueError(f"kernel must be one of {sorted(kinds)}")
    count = len(As)
    Ms, Ns, Ks = [], [], []
    for A, B in zip(As, Bs):
        _require_gpu_tensor(A, torch.float32, "A")
        _require_gpu_tensor(B, torch.float32, "B")
        M, K = (A.shape[1], A.shape[0]) if transA else (A.shape[0], A.shape[1])
        K2, N = (B.shape[1], B.shape[0]) if transB else (B.shape[0], B.shape[1])
        if K != K2:
            raise ValueError("inner dimensions differ")
        Ms.append(M); Ns.append(N); Ks.append(K)
    if Ds is None:
        Ds = [torch.empty((M, N), dtype=torch.float32, device=As[0].device) for M, N in zip(Ms, Ns)]
    for t in list(As) + list(Bs) + list(Ds) + list(Cs or []):
        if t.stride(1) != 1:
            raise ValueError("row-major tensors required")
    i32 = ctypes.c_int32 * count
    i64 = ctypes.c_int64 * count
    vp = ctypes.c_void_p * count
    need = L.lib().shampoo4_gemm_workspace_bytes(count)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=As[0].device)
    C_ptrs = vp(*[_ptr(c) for c in Cs]) if Cs else None
    C_ld = i64(*[c.stride(0) for c in Cs]) if Cs else None
    L.check(L.lib().shampoo4_gemm_batched_ex(
        kinds[kernel], count, int(transA), int(transB), i32(*Ms), i32(*Ns), i32(*Ks), alpha,
        vp(*[_ptr(a) for a in As]), i64(*[a.stride(0) for a in As]),
        vp(*[_ptr(b) for b in Bs]), i64(*[b.stride(0) for b in Bs]), beta, C_ptrs, C_ld,
        vp(*[_ptr(d) for d in Ds]), i64(*[d.stride(0) for d in Ds]),
        _ptr(workspace), workspace.numel(), _stream_ptr(stream)), "shampoo4_gemm_batched_ex")
    return Ds, workspace


def inverse_root(As, eps: float = 1e-6, iters: int = 20, Xs=None, workspace: torch.Tensor | None = None,
                 stream=None):
    """(A_i + eps I)^(-1/4) by the coupled Newton iteration on the MFMA GEMM (square,
    row-major fp32 device tensors).  Returns (Xs, workspace)."""
    count = len(As)
    for A in As:
        _require_gpu_tensor(A, torch.float32, "A")
        if A.dim() != 2 or A.shape[0] != A.shape[1] or (A.stride(1) != 1 and A.shape[1] > 1):
            raise ValueError("square row-major matrices required")
    ps = [int(A.shape[0]) for A in As]
    if Xs is None:
        Xs = [torch.empty((n, n), dtype=torch.float32, device=As[0].device) for n in ps]
    i32 = ctypes.c_int32 * count
    i64 = ctypes.c_int64 * count
    vp = ctypes.c_void_p * count
    parr = i32(*ps)
    need = L.lib().shampoo4_inverse_root_workspace_bytes(count, parr)
    if workspace is None or workspace.numel() < need:
        workspace = torch.empty(need, dtype=torch.uint8, device=As[0].device)
    L.check(L.lib().shampoo4_inverse_root(
        count, parr, vp(*[_ptr(a) for a in As]), i64(*[max(a.stride(0), a.shape[1]) for a in As]),
        float(eps), int(iters), vp(*[_ptr(x) for x in Xs]), i64(*[max(x.stride(0), x.shape[1]) for x in Xs]),
        _ptr(workspace), workspace.numel(), _stream_ptr(stream)), "shampoo4_inverse_root")
    return Xs, workspace
