"""The dequantize-to-bf16 path (oracle; test infrastructure only).

The abstract of "Realizing Native INT8 Compute for Diffusion Transformers on
Consumer GPUs" (arXiv 2606.14598) describes the shipped int8 forward that the
fused kernel replaces: weights and activations are quantized and then immediately
dequantized back to bf16, and a bf16 matrix multiply runs on the result.
Reading taken for the dequantization: v = bf16(fl32(float(q) * s)), i.e. the
fp32 product of the code and its row scale, rounded to bf16 (nearest even) —
what a plain ``(q.float() * s).to(bfloat16)`` computes.  The bf16 matrix
multiply is taken as exact (fp64 here) followed by the bias; a GPU bf16 GEMM
accumulates in fp32, so it is compared with a tolerance.
"""
from __future__ import annotations

import numpy as np

from .quant import bf16_to_f32, f32_to_bf16_bits, quantize_rows_ref


def dequant_rows_ref(q, s) -> np.ndarray:
    """q int8 [R,K], s fp32 [R] -> uint16 bf16 bits of fl32(float(q) * s[row])."""
    q = np.asarray(q, dtype=np.int8)
    s = np.asarray(s, dtype=np.float32)
    return f32_to_bf16_bits(q.astype(np.float32) * s[:, None])


def dequant_bf16_linear_ref(x, wq, s_w, bias=None) -> dict:
    """The whole slow path for bf16 x [M,K] and stored int8 weights wq [N,K]
    with scales s_w [N]: per-token quantization of x, dequantization of both
    operands to bf16, their product in fp64 plus the bias.  Returns xq, s_a,
    xd, wd (bf16 bits) and y64."""
    xq, s_a = quantize_rows_ref(x)
    xd = dequant_rows_ref(xq, s_a)
    wd = dequant_rows_ref(wq, s_w)
    y64 = bf16_to_f32(xd).astype(np.float64) @ bf16_to_f32(wd).astype(np.float64).T
    if bias is not None:
        y64 = y64 + bf16_to_f32(bias).astype(np.float64)[None, :]
    return dict(xq=xq, s_a=s_a, xd=xd, wd=wd, y64=y64)
