"""CPU oracle of the weight-quantized mixed-precision matmul.

TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the CPU
baseline leg of the benchmark may import this package; the library and its
Python binding never do, and nothing here is a fallback for the GPU path.
It shares no code with the GPU path.
"""
from .core import (  # noqa: F401
    unpack_weights, dequantize, k_part_bounds, qgemm_ref, qgemm_ref_kparts,
    round_fp16, fp16_within_tol, group_index, FP16_ATOL, FP16_RTOL, quantize_rows, qgemm_ref_scaled,
)
