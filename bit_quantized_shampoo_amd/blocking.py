"""Host-side parameter blocking with diagonal fallbacks.

Follows "Shampoo -- Second-Order Optimizer", section "Blocked and distributed variants":
every matrix parameter is cut into tiles of at most ``block`` x ``block`` that are
preconditioned independently (capping both the factor memory and the cubic cost), and
the page's two fallbacks:

* a tile dimension above the threshold ``max_dim`` (blocking off, ``block=None``, or
  tiles larger than the threshold): that side's factor is dropped and the tile keeps
  diagonal AdaGrad along it, the library's diagonal side (``Shampoo4Blocks(...,
  diagonal=block_diagonal_sides(plans))``), up to the library's limit ``max_diag_dim``
  for such a side; a parameter beyond that goes to the caller's diagonal method whole;
* 1-D (and 0-D) parameters such as biases and normalization gains stay on the caller's
  diagonal method (kind "diagonal").

Matrix parameters of higher rank (convolution kernels [out, in, kh, kw]) are viewed as
[out, in * kh * kw].  Tiles are row-major with a remainder tile at the end of each row
and column of tiles.  Everything here is host bookkeeping: the blocks are strided views
of the caller's tensors (no copies), which the library reads with their leading
dimensions.
"""

from __future__ import annotations

from dataclasses import dataclass, field


@dataclass
class ParamPlan:
    index: int                      # position in the caller's parameter list
    shape: tuple                    # the parameter's own shape
    kind: str                       # "blocks" or "diagonal"
    matrix: tuple | None = None     # (m, n) 2-D view for "blocks"
    tiles: list = field(default_factory=list)   # (r0, c0, rows, cols)
    tile_diagonal: list = field(default_factory=list)   # per tile (side L diagonal, side R diagonal)


def matrix_view_shape(shape) -> tuple | None:
    """[out, prod(rest)] for parameters of rank >= 2, None otherwise."""
    if len(shape) < 2:
        return None
    n = 1
    for d in shape[1:]:
        n *= int(d)
    return (int(shape[0]), n)


def tile(m: int, n: int, block: int) -> list:
    return [(r0, c0, min(block, m - r0), min(block, n - c0))
            for r0 in range(0, m, block) for c0 in range(0, n, block)]


def plan_blocks(shapes, block: int | None = 1024, max_dim: int = 8192, max_diag_dim: int = 65536) -> list:
    """One ParamPlan per parameter shape.  A tile side longer than ``max_dim`` is
    diagonal; a parameter whose diagonal side would exceed ``max_diag_dim`` goes to the
    caller's diagonal method whole."""
    if block is not None and block < 1:
        raise ValueError("block must be positive")
    if not 1 <= max_dim <= max_diag_dim:
        raise ValueError("need 1 <= max_dim <= max_diag_dim")
    out = []
    for i, shape in enumerate(shapes):
        shape = tuple(int(d) for d in shape)
        mv = matrix_view_shape(shape)
        if mv is None or 0 in mv:
            out.append(ParamPlan(i, shape, "diagonal"))
            continue
        m, n = mv
        tiles = [(0, 0, m, n)] if block is None else tile(m, n, block)
        if any(t[2] > max_diag_dim or t[3] > max_diag_dim for t in tiles):
            out.append(ParamPlan(i, shape, "diagonal"))
            continue
        diag = [(t[2] > max_dim, t[3] > max_dim) for t in tiles]
        out.append(ParamPlan(i, shape, "blocks", mv, tiles, diag))
    return out


def block_shapes(plans) -> list:
    """(rows, cols) of every tile, in plan order (the shapes a context is built for)."""
    return [(t[2], t[3]) for p in plans if p.kind == "blocks" for t in p.tiles]


def block_diagonal_sides(plans) -> list:
    """(side L diagonal, side R diagonal) of every tile, in block_shapes order."""
    return [d for p in plans if p.kind == "blocks" for d in p.tile_diagonal]


def block_views(tensors, plans) -> list:
    """Strided 2-D views of the tiles of `tensors` (same order as block_shapes)."""
    views = []
    for p in plans:
        if p.kind != "blocks":
            continue
        t = tensors[p.index]
        if not t.is_contiguous():
            raise ValueError(f"parameter {p.index} must be contiguous to be viewed as a matrix")
        mat = t.reshape(p.matrix)
        for (r0, c0, rows, cols) in p.tiles:
            views.append(mat[r0:r0 + rows, c0:c0 + cols])
    return views


def diagonal_indices(plans) -> list:
    return [p.index for p in plans if p.kind == "diagonal"]
