"""4-bit block codecs (linear-square and dynamic tree), bit-exact float32
emulation (oracle side).

TEST INFRASTRUCTURE ONLY -- see the package docstring.

Source: "4-bit Shampoo for Memory-Efficient Network Training", abstract.  The
page names linear-square quantization as the 4-bit codebook for the
eigenvector matrix and nothing more; the definition below is the reading
adopted here (every point is an interpretation, listed with its reason in the
design notes):

* Codebook.  Sixteen levels q_j = sign(t_j) * t_j**2 on the uniform grid
  t_j = -1 + 2j/15 (j = 0..15), except that q_7 is replaced by an exact 0 so
  that zeros (the identity's off-diagonal, all-zero blocks, padding) survive a
  round trip.  Times 225 the levels are the integers
  -225 -169 -121 -81 -49 -25 -9 0 1 9 25 49 81 121 169 225.
  Each level is stored as the float32 nearest the exact rational a_j / 225.
* Rounding.  Nearest level in the normalized domain, decided against float32
  midpoints m_j = RN32((a_j + a_{j+1}) / 450); a value equal to a midpoint
  takes the lower code.  code = number of midpoints strictly below x_hat.
* Blocks.  The matrix is flattened row-major and cut into blocks of
  ``qblock`` (64) consecutive elements; the last block is zero-padded.  The
  block scale is s = max |x| over the block (float32).  s == 0 gives code 7
  (the zero level) for the whole block.
* Normalization.  x_hat = RN32(x / s), an IEEE correctly rounded float32
  division (NumPy float32 division on x86 is exactly that, with subnormals
  kept).
* Packing.  Element 2i goes to the low nibble and element 2i+1 to the high
  nibble of byte i; a block therefore occupies qblock/2 bytes.
* Dequantization.  x = RN32(q[code] * s), one float32 multiply.

Parity status: pinned by tests (round trip on codebook values, identity
exactness, brute-force nearest-level search with exact rational distances,
hand-worked golden block).

Dynamic tree codebook (``codebook="dt"``).  The same abstract names dynamic tree
quantization as the alternative that linear-square slightly outperforms, and the
pages cite its source (the 8-bit optimizers paper) by title only; its definition is
taken from that published method and written out here (readings marked):

* A 4-bit pattern is a sign bit and three magnitude bits.  In the magnitude, the
  number E of leading zero bits is a base-10 exponent, the first one bit is an
  indicator, and the b = 2 - E bits after it are a linear fraction f: the value is
  sign * 10^-E * (1/10 + (9/10) * (2f + 1) / 2^(b+1)), i.e. the midpoints of 2^b
  equal bins of [1/10, 1], scaled into the decade [10^-(E+1), 10^-E].
* The all-zero magnitude is zero.  Reading: the pattern with the sign bit set and
  an all-zero magnitude (a second zero) stands for +1, so that the block maximum,
  which normalizes to exactly 1, is represented exactly -- as the linear-square
  codebook's top level does.
* Levels times 2000: -1775 -1325 -875 -425 -155 -65 -11 0 11 65 155 425 875 1325
  1775 2000.  Codes are indices into the ascending level list (the zero level is
  code 7 as in the linear-square codebook); rounding, midpoints, blocks,
  normalization, packing and dequantization are exactly as above.

Parity status of the dynamic tree levels: unpinned by the pages (the definition
is not on them); the tests pin the table to the bit-level decoding rule and the
nearest-level mechanics as for linear-square.
"""

from __future__ import annotations

from fractions import Fraction
from math import floor

import numpy as np

#: Codebook levels times 225 (integer numerators of the exact levels).
LEVEL_NUMERATORS = (-225, -169, -121, -81, -49, -25, -9, 0,
                    1, 9, 25, 49, 81, 121, 169, 225)
LEVEL_DENOMINATOR = 225
ZERO_CODE = 7


def rn32(value: Fraction) -> np.float32:
    """Round an exact rational to the nearest float32 (ties to even).

    Only normal-range magnitudes are needed here (the codebook lives in
    [2**-9, 1]); subnormal and overflow cases raise.
    """
    if value == 0:
        return np.float32(0.0)
    sign = -1 if value < 0 else 1
    mag = abs(value)
    e = mag.numerator.bit_length() - mag.denominator.bit_length() - 24
    two = Fraction(2)
    while mag / two ** e >= 2 ** 24:
        e += 1
    while mag / two ** e < 2 ** 23:
        e -= 1
    scaled = mag / two ** e
    n = floor(scaled)
    rem = scaled - n
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and n % 2 == 1):
        n += 1
    if not (-149 <= e and e + 24 <= 128):
        raise ValueError("rn32: value outside the normal float32 range")
    return np.float32(sign * n * 2.0 ** e)


def exact_levels() -> list[Fraction]:
    return [Fraction(a, LEVEL_DENOMINATOR) for a in LEVEL_NUMERATORS]


def exact_midpoints() -> list[Fraction]:
    lv = exact_levels()
    return [(lv[j] + lv[j + 1]) / 2 for j in range(15)]


#: float32 codebook and decision midpoints.
LEVELS = np.array([rn32(q) for q in exact_levels()], dtype=np.float32)
MIDPOINTS = np.array([rn32(m) for m in exact_midpoints()], dtype=np.float32)

LINEAR_SQUARE = "ls"
DYNAMIC_TREE = "dt"


def dynamic_tree_value(pattern: int) -> Fraction:
    """Exact value of a 4-bit dynamic tree pattern (bit 3: sign, bits 2..0: magnitude)."""
    if not 0 <= pattern < 16:
        raise ValueError("a 4-bit pattern")
    negative = bool(pattern & 8)
    mag = pattern & 7
    if mag == 0:
        return Fraction(1) if negative else Fraction(0)
    e = 3 - mag.bit_length()          # leading zeros of the 3-bit magnitude
    b = 2 - e                         # fraction bits after the indicator bit
    f = mag & ((1 << b) - 1)
    value = Fraction(1, 10 ** e) * (Fraction(1, 10) + Fraction(9, 10) * Fraction(2 * f + 1, 2 ** (b + 1)))
    return -value if negative else value


def exact_levels_of(codebook: str) -> list[Fraction]:
    if codebook == LINEAR_SQUARE:
        return exact_levels()
    if codebook == DYNAMIC_TREE:
        return sorted(dynamic_tree_value(t) for t in range(16))
    raise ValueError(f"unknown codebook {codebook!r}")


def _tables(codebook: str):
    lv = exact_levels_of(codebook)
    mids = [(lv[j] + lv[j + 1]) / 2 for j in range(15)]
    return (np.array([rn32(q) for q in lv], dtype=np.float32),
            np.array([rn32(m) for m in mids], dtype=np.float32))


_TABLES = {LINEAR_SQUARE: (LEVELS, MIDPOINTS), DYNAMIC_TREE: _tables(DYNAMIC_TREE)}


def levels(codebook: str = LINEAR_SQUARE) -> np.ndarray:
    """float32 levels (ascending) of a codebook."""
    return _TABLES[codebook][0]


def midpoints(codebook: str = LINEAR_SQUARE) -> np.ndarray:
    """float32 decision midpoints of a codebook."""
    return _TABLES[codebook][1]


def num_qblocks(n: int, qblock: int = 64) -> int:
    return (n + qblock - 1) // qblock


def quantize(x, qblock: int = 64, codebook: str = LINEAR_SQUARE):
    """Quantize a float32 array (flattened row-major) into packed 4-bit codes.

    Returns ``(codes, scales)``: ``codes`` is uint8 of length
    ``num_qblocks(n) * qblock // 2`` (padding codes are the zero code),
    ``scales`` is float32 of length ``num_qblocks(n)``.
    """
    x = np.ascontiguousarray(x, dtype=np.float32).ravel()
    n = x.size
    nqb = num_qblocks(n, qblock)
    padded = np.zeros(nqb * qblock, dtype=np.float32)
    padded[:n] = x
    blocks = padded.reshape(nqb, qblock)
    scales = np.max(np.abs(blocks), axis=1).astype(np.float32)
    codes = np.full(blocks.shape, ZERO_CODE, dtype=np.uint8)
    nz = scales > 0
    if np.any(nz):
        with np.errstate(invalid="ignore", divide="ignore", over="ignore"):
            xhat = (blocks[nz] / scales[nz, None]).astype(np.float32)
        codes[nz] = np.searchsorted(midpoints(codebook), xhat, side="left").astype(np.uint8)
    return pack_nibbles(codes.ravel()), scales


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    codes = np.asarray(codes, dtype=np.uint8).ravel()
    if codes.size % 2:
        codes = np.concatenate([codes, np.array([ZERO_CODE], np.uint8)])
    lo = codes[0::2] & 0xF
    hi = codes[1::2] & 0xF
    return (lo | (hi << 4)).astype(np.uint8)


def unpack_nibbles(packed: np.ndarray) -> np.ndarray:
    packed = np.asarray(packed, dtype=np.uint8).ravel()
    out = np.empty(packed.size * 2, dtype=np.uint8)
    out[0::2] = packed & 0xF
    out[1::2] = packed >> 4
    return out


def dequantize(codes, scales, n: int, qblock: int = 64, codebook: str = LINEAR_SQUARE) -> np.ndarray:
    """Inverse of :func:`quantize`: float32 array of length ``n``."""
    scales = np.asarray(scales, dtype=np.float32).ravel()
    c = unpack_nibbles(codes)
    nqb = scales.size
    c = c[: nqb * qblock].reshape(nqb, qblock)
    x = (levels(codebook)[c] * scales[:, None]).astype(np.float32)
    return x.ravel()[:n]


def quantize_matrix(U, qblock: int = 64, codebook: str = LINEAR_SQUARE):
    U = np.asarray(U, dtype=np.float32)
    return quantize(U.ravel(), qblock, codebook)


def dequantize_matrix(codes, scales, p: int, qblock: int = 64, codebook: str = LINEAR_SQUARE) -> np.ndarray:
    return dequantize(codes, scales, p * p, qblock, codebook).reshape(p, p)
