"""Dequantizing epilogue and the whole linear (oracle; test infrastructure only).

The abstract of "Realizing Native INT8 Compute for Diffusion Transformers on
Consumer GPUs" (arXiv 2606.14598) folds the per-token x per-channel
dequantization and the bias into the GEMM epilogue, which emits bf16.  Reading
taken: y[m,n] = (float(acc[m,n]) * s_a[m]) * s_w[n] + float(b[n]), evaluated
left to right in fp32 with every operation rounded separately (no fused
multiply-add), then rounded to bf16 (nearest even).  The fp64 evaluation of the
same expression is kept as the error-analysis reference.
"""
from __future__ import annotations

import numpy as np
from scipy.special import erfc

from .gemm import int_gemm_ref
from .quant import bf16_to_f32, f32_to_bf16_bits, quantize_rows_ref


def dequant_ref(acc, s_a, s_w, bias=None) -> np.ndarray:
    """fp32 epilogue: ((float(acc) * s_a[m]) * s_w[n]) + b[n], each op rounded."""
    acc = np.asarray(acc)
    s_a = np.asarray(s_a, dtype=np.float32)
    s_w = np.asarray(s_w, dtype=np.float32)
    t = acc.astype(np.float32) * s_a[:, None]
    y = t * s_w[None, :]
    if bias is not None:
        b = bf16_to_f32(bias) if not isinstance(bias, np.ndarray) or bias.dtype != np.float32 else bias
        y = y + b[None, :]
    return y.astype(np.float32)


def dequant_ref64(acc, s_a, s_w, bias=None) -> np.ndarray:
    """The same expression in fp64 (the scales and bias are exact in fp64)."""
    y = (np.asarray(acc).astype(np.float64) * np.asarray(s_a, np.float64)[:, None]) \
        * np.asarray(s_w, np.float64)[None, :]
    if bias is not None:
        b = bf16_to_f32(bias) if not isinstance(bias, np.ndarray) or bias.dtype != np.float32 else bias
        y = y + b.astype(np.float64)[None, :]
    return y


def w8a8_linear_ref(x, w, bias=None, wq=None, s_w=None) -> dict:
    """Whole fused W8A8 linear for bf16 x [M,K], w [N,K], bias [N] (or None).

    Passing ``wq``/``s_w`` skips the weight quantization (pre-quantized weights).
    Returns every intermediate: xq, s_a, wq, s_w, acc (int32), y32, y64 and
    y_bf16 (uint16 bits of bf16(y32)).
    """
    xq, s_a = quantize_rows_ref(x)
    if wq is None:
        wq, s_w = quantize_rows_ref(w)
    acc = int_gemm_ref(xq, wq, "i32")
    y32 = dequant_ref(acc, s_a, s_w, bias)
    y64 = dequant_ref64(acc, s_a, s_w, bias)
    return dict(xq=xq, s_a=s_a, wq=wq, s_w=s_w, acc=acc, y32=y32, y64=y64,
                y_bf16=f32_to_bf16_bits(y32))


def gelu_ref(y) -> np.ndarray:
    """Exact (erf) GELU, y * Phi(y) = 0.5 * y * (1 + erf(y / sqrt(2))), in fp64,
    evaluated as 0.5 * y * erfc(-y / sqrt(2)) so that the tail y << 0 keeps its
    relative accuracy (1 + erf cancels there)."""
    y = np.asarray(y, dtype=np.float64)
    return 0.5 * y * erfc(-y / np.sqrt(2.0))
