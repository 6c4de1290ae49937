"""Seeded synthetic inputs for the dense-and-sparse quantized GEMV.

This package only draws random numbers and arranges them into arrays of the
shapes, value laws and sparsity structure of the workloads.  It performs no
step of the method itself (no outlier selection, quantization, packing of
codes, decoding or matrix-vector product).  The one serialisation it does is
for the prefix-coded storage format: drawn integers are written as the
codewords of a fixed synthetic code (no code is fitted to data and no weight
is quantized), because a random byte string is not a stream of whole rows.
Both the CPU oracle (under
``oracle/``) and the GPU path's tests and benchmark take their inputs from
here, and from nowhere else.
"""

from .gen import (  # noqa: F401
    WORKLOADS,
    Workload,
    workload,
    layer_shape,
    make_weights,
    make_x,
    make_format_inputs,
    outlier_count,
    hptq_synthetic_code,
)
