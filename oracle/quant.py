"""Row-wise absmax int8 quantizer (oracle; test infrastructure only).

Follows the abstract of "Realizing Native INT8 Compute for Diffusion
Transformers on Consumer GPUs" (arXiv 2606.14598): activations are quantized
per token and weights per channel, and both scales are later folded into the
GEMM epilogue.  A token is a row of X [M,K]; a channel is a row of W [N,K]
(an output channel, the only weight granularity that factors out of the sum
over K).  The same row quantizer therefore serves both.

Readings taken where the pages are silent:
  * scale s = fl32(amax / 127) with amax = max_k |v[k]| (symmetric, no zero point);
  * q[k] = clamp(rne(fl32(v[k] / s)), -127, 127): the quotient is the correctly
    rounded fp32 division, then rounded half-to-even to an integer;
  * an all-zero row gets s = 0 and q = 0 (no 0/0).
All arithmetic is IEEE fp32, the precision the quantized codes are decided in.
"""
from __future__ import annotations

import numpy as np
import torch


def bf16_to_f32(x) -> np.ndarray:
    """bf16 (torch tensor, or uint16 bit patterns) -> float32, exactly."""
    if isinstance(x, torch.Tensor):
        bits = x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)
    else:
        bits = np.asarray(x, dtype=np.uint16)
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(y) -> np.ndarray:
    """float32 -> bf16 bit patterns, round to nearest even (torch's CPU cast)."""
    t = torch.from_numpy(np.ascontiguousarray(y, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def quantize_rows_ref(v) -> tuple[np.ndarray, np.ndarray]:
    """Quantize each row of ``v`` [R,K] to int8 with its own fp32 scale.

    Returns (q int8 [R,K], s float32 [R]).  ``v`` is a bf16 torch tensor or a
    float32 array holding bf16-representable values.
    """
    if isinstance(v, torch.Tensor):
        v = bf16_to_f32(v)
    v = np.asarray(v, dtype=np.float32)
    if v.ndim != 2:
        raise ValueError("expected a 2-D [rows, K] array")
    R, K = v.shape
    if K == 0:
        return np.zeros((R, 0), np.int8), np.zeros(R, np.float32)
    amax = np.max(np.abs(v), axis=1)                  # exact
    s = amax / np.float32(127.0)                      # fp32, correctly rounded
    q = np.zeros((R, K), dtype=np.int8)
    nz = amax != 0
    quot = v[nz] / s[nz, None]                        # fp32 quotient, correctly rounded
    q[nz] = np.clip(np.rint(quot), -127, 127).astype(np.int8)   # rint: half to even
    s = np.where(nz, s, np.float32(0.0)).astype(np.float32)
    return q, s
