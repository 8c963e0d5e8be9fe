"""The five synthetic workloads (shapes, distributions, schedule).

Every gradient is drawn from NumPy's ``default_rng`` seeded by a
``SeedSequence`` keyed on (seed, source matrix) for fixed per-matrix factors
and on (seed, step, source matrix) for per-step noise, so any step of any
block can be regenerated on its own.  Large source matrices are cut into
blocks of order at most 1024 (tiles of 1024 plus a remainder, row-major), the
blocking the Shampoo blog page describes in "Blocked and distributed
variants".

Workloads (names describe what they are):

* ``single_64x32``      one [64, 32] block, anisotropic rows/columns,
                        20 steps, root refresh every step.
* ``single_1024``       one [1024, 1024] block, same generator, 100 steps,
                        root refresh every 10 steps.
* ``cnn_batch``         50 conv-like matrices drawn from
                        {[64,576], [128,1152], [256,2304], [512,4608]},
                        lognormal column scales, split into <=1024 blocks.
* ``transformer_batch`` 24 layers x {QKV [3072,1024], O [1024,1024],
                        FFN-up [4096,1024], FFN-down [1024,4096]} = 288
                        blocks of [1024,1024]; Student-t(3) entries rounded
                        to bfloat16 and widened back to float32.
* ``large_4096``        64 blocks of [4096, 4096], rank-32 signal plus noise,
                        5 Bjorck iterations.
"""

from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

BLOCK_CAP = 1024


def split_blocks(m: int, n: int, cap: int = BLOCK_CAP):
    """Row-major list of (r0, c0, rows, cols) tiles of order <= cap."""
    tiles = []
    for r0 in range(0, m, cap):
        for c0 in range(0, n, cap):
            tiles.append((r0, c0, min(cap, m - r0), min(cap, n - c0)))
    return tiles


def round_to_bf16(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 (ties to even) -> float32."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    bits = x.view(np.uint32).astype(np.uint64)
    bits = (bits + 0x7FFF + ((bits >> 16) & 1)) & 0xFFFF0000
    return bits.astype(np.uint32).view(np.float32)


@dataclass
class Workload:
    name: str
    description: str
    sources: list            # source matrix shapes (m, n)
    kind: str                # generator kind
    beta: float = 0.95
    eps: float = 1e-6
    qblock: int = 64
    bjorck_iters: int = 1
    power_iters: int = 1
    root_interval: int = 1
    steps: int = 10
    seed: int = 0
    block_cap: int = BLOCK_CAP   # largest block order after splitting
    blocks: list = field(default_factory=list)   # (source, r0, c0, m, n)

    def __post_init__(self):
        self.blocks = []
        for s, (m, n) in enumerate(self.sources):
            for (r0, c0, bm, bn) in split_blocks(m, n, self.block_cap):
                self.blocks.append((s, r0, c0, bm, bn))

    @property
    def shapes(self):
        return [(bm, bn) for (_, _, _, bm, bn) in self.blocks]

    # -- per-source fixed factors -----------------------------------------
    def _fixed(self, s: int):
        m, n = self.sources[s]
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, 1_000_003, s]))
        if self.kind == "aniso":
            a = rng.uniform(-1.0, 1.0, size=m)
            b = rng.uniform(-1.0, 1.0, size=n)
            return (10.0 ** a)[:, None] * (10.0 ** b)[None, :]
        if self.kind == "conv":
            return rng.lognormal(0.0, 1.0, size=n)[None, :]
        if self.kind == "lowrank":
            A = rng.standard_normal((m, 32))
            B = rng.standard_normal((n, 32))
            return (A, B)
        return None

    def source_gradient(self, s: int, step: int) -> np.ndarray:
        """Full source gradient ``s`` at ``step`` (float32)."""
        m, n = self.sources[s]
        fixed = self._fixed(s)
        rng = np.random.default_rng(np.random.SeedSequence([self.seed, step, s]))
        if self.kind == "aniso":
            G = rng.standard_normal((m, n)) * fixed
        elif self.kind == "conv":
            G = rng.standard_normal((m, n)) * fixed
        elif self.kind == "student_bf16":
            G = round_to_bf16(rng.standard_t(3.0, size=(m, n)).astype(np.float32))
        elif self.kind == "lowrank":
            A, B = fixed
            Z = rng.standard_normal((32, 32))
            G = (A @ Z @ B.T) / 32.0 + 0.01 * rng.standard_normal((m, n))
        else:
            raise ValueError(self.kind)
        return np.ascontiguousarray(G, dtype=np.float32)

    def gradients(self, step: int):
        """List of per-block float32 gradients at ``step`` (contiguous copies)."""
        cache = {}
        out = []
        for (s, r0, c0, bm, bn) in self.blocks:
            if s not in cache:
                cache[s] = self.source_gradient(s, step)
            out.append(np.ascontiguousarray(cache[s][r0:r0 + bm, c0:c0 + bn]))
        return out

    def block_gradient(self, b: int, step: int) -> np.ndarray:
        s, r0, c0, bm, bn = self.blocks[b]
        return np.ascontiguousarray(self.source_gradient(s, step)[r0:r0 + bm, c0:c0 + bn])


def _cnn_sources(seed: int, count: int = 50):
    shapes = [(64, 576), (128, 1152), (256, 2304), (512, 4608)]
    rng = np.random.default_rng(np.random.SeedSequence([seed, 7]))
    idx = rng.integers(0, len(shapes), size=count)
    return [shapes[i] for i in idx]


def _transformer_sources(layers: int = 24):
    src = []
    for _ in range(layers):
        src += [(3072, 1024), (1024, 1024), (4096, 1024), (1024, 4096)]
    return src


def _make(name: str) -> Workload:
    if name == "single_64x32":
        return Workload(name, "one [64,32] block, N(0,1) scaled per row by 10^U(-1,1) and per "
                        "column by 10^U(-1,1); beta 0.95, eps 1e-6, 4-bit blocks of 64, "
                        "root refresh every step, 20 steps, seed 0",
                        [(64, 32)], "aniso", steps=20, root_interval=1)
    if name == "single_1024":
        return Workload(name, "one [1024,1024] fp32 block, same anisotropic generator; stats "
                        "every step, root refresh every 10 steps, 100 steps",
                        [(1024, 1024)], "aniso", steps=100, root_interval=10)
    if name == "cnn_batch":
        return Workload(name, "50 conv-like matrices from {[64,576],[128,1152],[256,2304],"
                        "[512,4608]} split into <=1024-order blocks; N(0,1) x lognormal(0,1) "
                        "column scales", _cnn_sources(0), "conv", steps=10)
    if name == "transformer_batch":
        return Workload(name, "24 layers x {QKV [3072,1024], O [1024,1024], FFN-up [4096,1024], "
                        "FFN-down [1024,4096]} split into 288 [1024,1024] blocks; Student-t(3) "
                        "entries rounded to bf16, widened to fp32",
                        _transformer_sources(), "student_bf16", steps=10)
    if name == "large_4096":
        return Workload(name, "64 blocks of [4096,4096]: rank-32 signal A Z B^T/32 plus 0.01 "
                        "N(0,1) noise; 5 Bjorck iterations, root refresh every step",
                        [(4096, 4096)] * 64, "lowrank", bjorck_iters=5, steps=3,
                        block_cap=4096)
    raise KeyError(name)


CONFIGS = ["single_64x32", "single_1024", "cnn_batch", "transformer_batch", "large_4096"]


def get_workload(name: str) -> Workload:
    return _make(name)
