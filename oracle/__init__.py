"""CPU oracle for block-scaled FP8 / NVFP4 (grouped) GEMM.

TEST INFRASTRUCTURE ONLY.  Only the test suite, the package's smoke check and
the benchmark's CPU-baseline leg import this package.  The GPU library never
calls it, links it or falls back to it, and this package shares no code,
table or helper with the HIP path: it decodes the stored formats itself from
their bit-field definitions and computes in float64 with NumPy.

What it computes (the plain definition of the result; the kernels reach the
same value up to FP32 rounding order and the final BF16 rounding):

  grouped FP8   C[i, n] = sum_kb a_scale[i, kb] * b_scale[g, n // 128, kb]
                          * sum_{k in kb} e4m3(A[i, k]) * e4m3(B[g, n, k]),
                g = m_indices[i]; rows with g = -1 are exactly zero.
                (flashinfer#7877 page, "Intro" and "Code analysis 1": E4M3
                inputs, rows grouped by m_indices, FP32 per-128 block scales,
                BF16 output; kernel argument list A, B, C, a_scale, b_scale,
                m_indices, M, N, K, G.)
  NVFP4         C[i, n] = alpha * sum_k (e2m1(A[i, k]) * e4m3(sA[i, k // 16]))
                                    * (e2m1(B[n, k]) * e4m3(sB[n, k // 16])),
                alpha = gA * gB; grouped: B[g], sB[g] with g = m_indices[i].
                (onnxruntime#29824 page, "Code analysis 1": W4A4 grouped GEMM
                for MoE prefill; flashinfer#3948 page: dense mm_fp4.)

  quantisers   oracle.quant: BF16 activations -> FP8 E4M3FN codes with one
                FP32 scale per row and 128-wide K block, and -> NVFP4 (E2M1
                codes, E4M3 scale per 16 elements, FP32 global scale); see
                that module for the definition and its precision.

Pins: the test suite checks these functions against exhaustive format
tables, exact integer / rational brute force, hand-computed worked examples
and invariants.  Parity status of each function is stated in its docstring.
"""
from .formats import (  # noqa: F401
    decode_e4m3fn,
    decode_e2m1,
    unpack_e2m1,
    bf16_rne_bits,
    bf16_bits_to_float,
)
from .gemm import (  # noqa: F401
    grouped_fp8_gemm,
    fp4_gemm,
    grouped_fp4_gemm,
    fp4_gemm_problems,
    grouped_w4a16_gemm,
    rms_nonpadding,
    check_tolerance,
)
