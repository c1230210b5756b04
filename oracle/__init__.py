"""CPU oracle for D = alpha*op(A)@op(B) + beta*C (test infrastructure only).

Only tests, the package smoke check and the benchmark's CPU-baseline leg may
import this package. It shares no code with the HIP library.
"""
from .gemm_oracle import (  # noqa: F401
    F16, BF16, F8E4M3, F8E5M2, RTOL, ATOL, decode_fp8,
    round_f32_to_f16_bits, round_f32_to_bf16_bits, round_f32_bits, decode_bits,
    op_a, op_b, c_matrix, gemm_reference, gemm_reference_f32, gemm_reference_i8,
    gemm_reference_elements, check,
)
