"""CPU oracle for the FP8 block-scaled NT GEMM (test infrastructure only).

This package is the slow, plain reference that the GPU library is checked
against.  It is test infrastructure: only the tests, the smoke check and the
CPU-baseline leg of the benchmark may import it.  The GPU library never calls
it, and it shares no code with the GPU library.

What it computes comes from the DeepGEMM pages:

* "DeepSeek open-source week day 3" (deepseek.csdn.net), section
  "technical features": FP8 operands with fine-grained dynamic scaling and a
  second, higher-precision accumulation level above the FP8 tensor-core sums;
  the contiguous and masked MoE grouped layouts.
* "DeepGEMM: making LLM matrix multiplication fly" (pomoai.com), section
  "core functions": block-wise scaling, each small block scaled on its own;
  section "technical details": the ``fp8_gemm_nt`` naming (D = A . B^T with
  both operands K-contiguous).

The pages leave the granularity, the fp8 variant and the output type open.
The readings taken here: A carries one fp32 scale per 1x128 K-slice, B one
per 128x128 block, fp8 is OCP e4m3 (max 448), scale = amax/448, and D is
bf16.  Every reading is listed with its reason in the design notes.

Modules
-------
e4m3   exact 256-entry decode table, round-to-nearest-even saturating encoder
e2m1   the FP4 codec (16 codes) and its two-per-byte packing
quant  1x128 (activation) and 128x128 (weight) quantisers, FP8 and FP4
gemm   dense, contiguous-grouped, masked-grouped and K-grouped reference GEMMs in fp64,
       the BF16 and FP4 NT GEMMs; FC1 + SwiGLU on the masked and contiguous layouts
check  the element-wise acceptance rule
"""

from .e4m3 import E4M3_MAX, decode_table, decode, encode  # noqa: F401
from .quant import quantize_a_1x128, quantize_b_128x128  # noqa: F401
from .quant import quantize_a_1x128_fp4, quantize_b_128x128_fp4  # noqa: F401
from .gemm import (  # noqa: F401
    gemm_nt_ref,
    gemm_nt_ref_at,
    grouped_contiguous_ref,
    grouped_masked_ref,
    k_grouped_ref,
    k_grouped_ref_at,
    bf16_gemm_nt_ref,
    bf16_to_f64,
    fp4_gemm_nt_ref,
    masked_swiglu_quant_ref,
    masked_swiglu_ref,
    contiguous_swiglu_quant_ref,
    contiguous_swiglu_ref,
    silu,
)
from .check import tolerance_check, bf16_bits_to_float, bf16_round  # noqa: F401
