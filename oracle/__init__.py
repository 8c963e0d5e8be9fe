"""CPU oracle for the 4-bit Shampoo preconditioner step.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call or
link anything in this package: only ``tests/``, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code, table or
constant with the HIP implementation in ``bit_quantized_shampoo_amd``.

It is deliberately plain and slow: NumPy float64 for every matrix operation,
a bit-exact float32 emulation for the 4-bit codec, one matrix at a time, in
the order the method's steps are described.

Sources (web pages, cited by title and section):

* "4-bit Shampoo for Memory-Efficient Network Training" (Wang, Zhou, Li,
  Huang; arXiv 2405.18144), abstract: second-order states kept in 4 bits by
  quantizing the eigenvector matrix of the preconditioner rather than the
  preconditioner; orthogonality of the quantized eigenvector matrix is
  rectified before use, also for the inverse 4th root; linear-square
  quantization is the codebook.
* "Shampoo — Second-Order Optimizer" (aicassindra.com blog): sections
  "Kronecker factorization", "Where the fourth root comes from",
  "Rotation, not just rescaling", "Computing the inverse fourth root",
  "The cost dial", "Pitfalls, and the small-model view".

Modules:

* ``codec``      -- linear-square 4-bit block codec (bit-exact float32).
* ``shampoo4``   -- the preconditioner step (float64 matrix math).
* ``bruteforce`` -- full-matrix (Kronecker / AdaGrad) constructions used only
                    to pin the oracle on tiny sizes.
"""

from . import codec, shampoo4, bruteforce  # noqa: F401
