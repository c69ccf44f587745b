"""The dequantize-to-bf16 path, kept as a measured comparator.

The abstract of "Realizing Native INT8 Compute for Diffusion Transformers on
Consumer GPUs" (arXiv 2606.14598) traces the slowness of the shipped int8
forward to this path: activations and weights are quantized to int8
and then immediately dequantized back to bf16 for a bf16 matrix multiply, so
the int8 matrix units are never used.  ``dequant_bf16_linear`` reproduces it
on the same stored int8 weights as the fused path: per-token quantization
(libw8a8), dequantization of both operands (libw8a8), then a bf16 GEMM with
bias (torch ``F.linear``, hipBLASLt).  It is not the fused path.
"""
from __future__ import annotations

import torch

from .ops import dequantize_rows, quantize_act


def dequant_bf16_linear(x: torch.Tensor, wq: torch.Tensor, w_scale: torch.Tensor,
                        bias: torch.Tensor | None = None, scratch: dict | None = None) -> torch.Tensor:
    """bf16 x [M,K] and int8 weights wq [N,K] (scales w_scale [N]) -> bf16 y [M,N]
    through quantize -> dequantize -> bf16 GEMM.  ``scratch`` (a dict) keeps the
    intermediate buffers between calls."""
    s = scratch if scratch is not None else {}
    M, K = x.shape
    N = wq.shape[0]
    if s.get("shape") != (M, N, K):
        s.update(shape=(M, N, K),
                 xq=torch.empty((M, K), dtype=torch.int8, device=x.device),
                 xs=torch.empty((M,), dtype=torch.float32, device=x.device),
                 xd=torch.empty((M, K), dtype=torch.bfloat16, device=x.device),
                 wd=torch.empty((N, K), dtype=torch.bfloat16, device=x.device))
    quantize_act(x, s["xq"], s["xs"])
    dequantize_rows(s["xq"], s["xs"], s["xd"])
    dequantize_rows(wq, w_scale, s["wd"])
    return torch.nn.functional.linear(s["xd"], s["wd"], bias)
