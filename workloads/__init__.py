"""Seeded synthetic inputs for block-scaled FP8 / NVFP4 (grouped) GEMM.

This package is the single source of inputs for both the CPU oracle and the
HIP path.  It draws random matrices, routes rows to experts, and quantises the
matrices to the stored formats (E4M3FN codes with FP32 block scales, or NVFP4
packed E2M1 codes with E4M3 block scales and an FP32 global scale).  It holds
none of the GEMM's arithmetic: no decoding for a product, no accumulation, no
rescaling of partial sums.  Neither the oracle nor the HIP binding is imported
here, and this package imports neither.
"""
from .quant import (  # noqa: F401
    e4m3fn_encode,
    e2m1_encode,
    quantize_fp8_rows,
    quantize_fp8_blocks,
    quantize_nvfp4,
)
from .gen import (  # noqa: F401
    CONFIGS,
    make,
    fp8_problem,
    nvfp4_problem,
    w4a16_problem,
    decode_routing,
    runs_to_indices,
    moe_expand,
    bf16_activations,
)
