"""4-bit Shampoo preconditioner step for MI355X (gfx950).

The computation lives in ``libshampoo4.so`` (hand-written HIP kernels behind
the C ABI in ``include/shampoo4.h``); this package is its PyTorch-facing
binding.  Build with ``python -m bit_quantized_shampoo_amd.build``.
"""

from ._lib import LIB_PATH, Shampoo4Error  # noqa: F401
from .shampoo4 import (Shampoo4Blocks, Shampoo4Config, codebook, dequantize,  # noqa: F401
                       gemm_batched, inverse_root, plan, quantize)
