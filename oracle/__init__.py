"""CPU oracle for the fused W8A8 linear (per-token int8 activations x
per-output-channel int8 weights -> int32 -> bf16).

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call, link
or execute anything in this directory: only the tests, the package smoke entry
and the benchmark's CPU-baseline leg use it.  It shares no code with the HIP
library (no headers, helpers, tables or generators).

What it computes follows the abstract of "Realizing Native INT8 Compute for
Diffusion Transformers on Consumer GPUs: A Fused INT8 GEMM Kernel for Ideogram
4.0" (arXiv 2606.14598): weights and activations are quantized to int8, the
product is accumulated int8 x int8 -> int32, and a per-token x per-channel
dequantization plus the bias turn the int32 result into the bf16 output.  The
pages leave the scale formula, rounding and clamp open; the readings taken
here are absmax/127 scales in fp32, round-half-to-even on the fp32 quotient
and a clamp to [-127, 127].

Functions:
  quantize_rows_ref   row-wise absmax quantizer (tokens of X, output channels of W)
  int_gemm_ref        plain integer GEMM, int32 (wrap-around) or int64 accumulation
  dequant_ref         fp32 dequant + bias, evaluated in the stated order
  dequant_ref64       the same in fp64 (error-analysis reference)
  w8a8_linear_ref     the whole path, returning every intermediate
  gelu_ref            exact erf GELU in fp64 (glue of the MLP-pair workload)
  dequant_rows_ref    int8 codes x row scale -> bf16 (the dequantize-to-bf16 path)
  dequant_bf16_linear_ref  that whole path: quantize, dequantize, product in fp64
  quantize_rows_fp8_ref, fp8_gemm_ref, fp32_sum_bound, fp8_block_sum_bound, w8a8_fp8_linear_ref
                      the fp8 (e4m3) variant of the method (module oracle.fp8)
"""
from .quant import bf16_to_f32, f32_to_bf16_bits, quantize_rows_ref
from .gemm import int_gemm_ref
from .dequant import dequant_ref, dequant_ref64, w8a8_linear_ref, gelu_ref
from .slowpath import dequant_rows_ref, dequant_bf16_linear_ref
from .fp8 import (e4m3_decode, e4m3_encode, e4m3_round, fp32_sum_bound, fp8_block_sum_bound,
                  fp8_gemm_ref, quantize_rows_fp8_ref, w8a8_fp8_linear_ref)

__all__ = ["bf16_to_f32", "f32_to_bf16_bits", "quantize_rows_ref", "int_gemm_ref",
           "dequant_ref", "dequant_ref64", "w8a8_linear_ref", "gelu_ref",
           "dequant_rows_ref", "dequant_bf16_linear_ref", "e4m3_decode", "e4m3_encode",
           "e4m3_round", "fp32_sum_bound", "fp8_block_sum_bound", "fp8_gemm_ref", "quantize_rows_fp8_ref",
           "w8a8_fp8_linear_ref"]
