"""CPU oracle for the dense-and-sparse quantized GEMV -- TEST INFRASTRUCTURE ONLY.

This package is the plain, slow, fp64 statement of what the GPU path must
compute.  Only the test suite, the smoke check and the benchmark's CPU
baseline leg may import it; the product path (the C-ABI library and its
Python binding) never does, and shares no code, table or constant with it.

Contents, each following the pages it cites:

* ``encode``     -- outlier pick, uniform group quantization, sensitivity-
                    weighted Lloyd LUT, sparse residual in CSR.
* ``pack``       -- the canonical per-row LSB-first code bitstream.
* ``gemv``       -- decode and y = dequant(W_dense) x + W_sparse x in fp64,
                    and the per-output tolerance scale.
* ``accounting`` -- bits-per-weight of the format.

Sources ("the pages"):
  [SpQR]   "SpQR (Sparse-Quantized Representation)"
  [SqLLM]  "SqueezeLLM (Dense-and-Sparse Quantization)"
"""

from . import accounting, encode, gemv, pack  # noqa: F401
