"""Linear-square 4-bit block codec, bit-exact float32 emulation (oracle side).

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


def num_qblocks(n: int, qblock: int = 64) -> int:
    return (n + qblock - 1) // qblock


def quantize(x, qblock: int = 64):
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
        codes[nz] = np.searchsorted(MIDPOINTS, xhat, side="left").astype(np.uint8)
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


def dequantize(codes, scales, n: int, qblock: int = 64) -> np.ndarray:
    """Inverse of :func:`quantize`: float32 array of length ``n``."""
    scales = np.asarray(scales, dtype=np.float32).ravel()
    c = unpack_nibbles(codes)
    nqb = scales.size
    c = c[: nqb * qblock].reshape(nqb, qblock)
    x = (LEVELS[c] * scales[:, None]).astype(np.float32)
    return x.ravel()[:n]


def quantize_matrix(U, qblock: int = 64):
    U = np.asarray(U, dtype=np.float32)
    return quantize(U.ravel(), qblock)


def dequantize_matrix(codes, scales, p: int, qblock: int = 64) -> np.ndarray:
    return dequantize(codes, scales, p * p, qblock).reshape(p, p)
