"""Algorithmic work accounting (flops and bytes) for throughput reporting.

The page-level formulas come from "Shampoo -- Second-Order Optimizer",
sections "Kronecker factorization" (factor memory m^2 + n^2) and "The cost
dial" (statistics 2 m^2 n + 2 m n^2, applying both roots 2 m^2 n + 2 m n^2,
overhead ratio 2 (m + n) / (3 B) against a 6 B m n forward+backward).

The 4-bit step's own accounting (``side_flops`` and friends) counts every
matrix product as a full 2 M N K, symmetric or not, which is the page's
convention; the codec moves 4 + 1/2 + 4/qblock bytes per element
(fp32 value, one nibble, the block's fp32 scale).
"""

from __future__ import annotations


def page_step_flops(m: int, n: int) -> int:
    """Vanilla Shampoo per-step cost: statistics plus applying both roots."""
    return 2 * m * m * n + 2 * m * n * n + 2 * m * m * n + 2 * m * n * n


def page_overhead_ratio(m: int, n: int, batch_tokens: float) -> float:
    return 2.0 * (m + n) / (3.0 * batch_tokens)


def factor_floats(m: int, n: int) -> int:
    return m * m + n * n


def codec_bytes_per_element(qblock: int = 64) -> float:
    return 4.0 + 0.5 + 4.0 / qblock


# -- 4-bit step ---------------------------------------------------------------

def bjorck_flops(p: int, iters: int) -> float:
    """V^T V then V (V^T V): two p x p x p products per iteration."""
    return iters * 4.0 * p ** 3


def stats_flops(p: int, q: int) -> float:
    """V diag(lam) V^T (2 p^3) and the side's G G^T (2 p^2 q)."""
    return 2.0 * p ** 3 + 2.0 * p * p * q


def refresh_flops(p: int, power_iters: int = 1) -> float:
    """P = L~ V (2 p^3 per power step), Householder QR with explicit Q
    (4/3 p^3 + 4/3 p^3), Rayleigh product L~ Q (2 p^3)."""
    return power_iters * (2.0 * p ** 3 + (8.0 / 3.0) * p ** 3) + 2.0 * p ** 3


def precondition_side_flops(p: int, q: int) -> float:
    """Two of the four [p,p] x [p,q] products of the eigen-form sandwich."""
    return 4.0 * p * p * q


def block_step_flops(m: int, n: int, bjorck_iters: int, root_interval: int = 1,
                     power_iters: int = 1, cached_root: bool = True) -> float:
    """Algorithmic flops of one block-step (update_stats + amortized refresh_root +
    precondition).  With ``cached_root`` the rectified root eigenvectors are
    computed once per refresh and, when refreshing every step, shared with the
    next step's statistics update; otherwise every precondition rectifies them
    again."""
    total = 0.0
    for p, q in ((m, n), (n, m)):
        total += bjorck_flops(p, bjorck_iters)                # stats side
        total += stats_flops(p, q)
        total += refresh_flops(p, power_iters)
        total += precondition_side_flops(p, q)
        if cached_root:
            if root_interval > 1:
                total += bjorck_flops(p, bjorck_iters) / root_interval
        else:
            total += bjorck_flops(p, bjorck_iters)
    return total


def block_step_codec_bytes(m: int, n: int, qblock: int = 64) -> float:
    """One dequantize and one quantize of each side's eigenvector matrix."""
    per = codec_bytes_per_element(qblock)
    return 2.0 * per * (m * m + n * n)
