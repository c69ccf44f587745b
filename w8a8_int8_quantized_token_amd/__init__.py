"""MI355X-native fused W8A8 linear (per-token int8 activations x
per-output-channel int8 weights -> int32 on the matrix cores -> dequant +
bias epilogue -> bf16), a thin torch binding over libw8a8.so.

The method is the one in the abstract of "Realizing Native INT8 Compute for
Diffusion Transformers on Consumer GPUs: A Fused INT8 GEMM Kernel for
Ideogram 4.0" (arXiv 2606.14598).
"""
from ._lib import LIB_PATH, MAX_K, W8A8Error, lib, status_str
from .module import W8A8Linear
from .ops import (dequantize_rows, gemm_f32_fp8, gemm_i32, linear, linear_fp8, linear_splitk,
                  mfma_ceiling, num_tiles, select_splitk, splitk_workspace_bytes,
                  quantize_act, quantize_act_fp8, quantize_weight, quantize_weight_fp8,
                  select_tile, tile_info)
from .slowpath import dequant_bf16_linear

__all__ = ["LIB_PATH", "MAX_K", "W8A8Error", "W8A8Linear", "dequant_bf16_linear",
           "dequantize_rows", "gemm_f32_fp8", "gemm_i32", "lib", "linear", "linear_fp8", "linear_splitk",
           "mfma_ceiling", "select_splitk", "splitk_workspace_bytes",
           "num_tiles", "quantize_act", "quantize_act_fp8", "quantize_weight",
           "quantize_weight_fp8", "select_tile", "status_str", "tile_info"]
