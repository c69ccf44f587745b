"""W8A8 with fp8 (e4m3) codes instead of int8 (oracle; test infrastructure only).

The pages compare the int8 path against fp8 (and nf4) alternatives; this is
the fp8 variant of the same method on one GPU: activations quantized per
token and weights per output channel to the OCP e4m3 format (1 sign bit,
4 exponent bits with bias 7, 3 mantissa bits; largest finite value 448,
smallest normal 2^-6, subnormal spacing 2^-9), products accumulated in fp32,
and the same per-token x per-channel dequantization plus bias folded into the
epilogue.

Readings taken (the pages give no fp8 recipe):
  * scale s = fl32(amax / 448), the int8 recipe with 448 in place of 127;
  * code = e4m3 value nearest to fl32(v / s), ties to the even mantissa,
    saturating at +-448 (|v/s| <= 448 up to one fp32 rounding, so saturation
    only guards that rounding); an all-zero row gives s = 0 and zero codes;
  * the accumulation is exact here (fp64: every e4m3 x e4m3 product and every
    partial sum of K <= 133144 of them is representable).  A sequential fp32
    sum is within gamma_K * sum_k |x_k w_k| (gamma_K = K u / (1 - K u),
    u = 2^-24) of it (fp32_sum_bound).  A device that sums blocks of products
    at an internal precision below fp32 is held to fp8_block_sum_bound, which
    states its reading of that arithmetic.
"""
from __future__ import annotations

import numpy as np
import torch

from .dequant import dequant_ref
from .quant import bf16_to_f32, f32_to_bf16_bits

E4M3_MAX = 448.0


def e4m3_round(v) -> np.ndarray:
    """Nearest e4m3 value of each element (float64 in, float64 out), ties to
    the even mantissa, saturating at +-448."""
    v = np.asarray(v, dtype=np.float64)
    a = np.abs(v)
    out = np.zeros_like(a)
    sub = a < 2.0 ** -6
    out[sub] = np.rint(a[sub] * 2.0 ** 9) * 2.0 ** -9          # subnormal grid, rint: half to even
    nrm = ~sub
    e = np.floor(np.log2(np.where(nrm, a, 1.0)))
    # guard log2 rounding at exact powers of two
    e = np.where(2.0 ** e > a, e - 1, e)
    e = np.where(2.0 ** (e + 1) <= a, e + 1, e)
    spacing = 2.0 ** (e - 3)
    out[nrm] = (np.rint(a / spacing) * spacing)[nrm]
    out = np.minimum(out, E4M3_MAX)
    return np.copysign(out, v)


def e4m3_encode(val) -> np.ndarray:
    """e4m3 values (exactly representable) -> uint8 codes."""
    val = np.asarray(val, dtype=np.float64)
    sign = np.signbit(val).astype(np.uint8) << 7
    a = np.abs(val)
    code = np.zeros(a.shape, dtype=np.uint8)
    sub = a < 2.0 ** -6
    code[sub] = (a[sub] * 2.0 ** 9).astype(np.uint8)
    nrm = ~sub
    e = np.floor(np.log2(np.where(nrm, a, 1.0))).astype(np.int64)
    mant = np.where(nrm, a / 2.0 ** e * 8 - 8, 0).astype(np.int64)
    code[nrm] = ((e[nrm] + 7) << 3 | mant[nrm]).astype(np.uint8)
    return code | sign


def e4m3_decode(code) -> np.ndarray:
    """uint8 e4m3 codes -> float64 values (0x7F / 0xFF, NaN, are never produced)."""
    c = np.asarray(code, dtype=np.uint8).astype(np.int64)
    s = np.where(c & 0x80, -1.0, 1.0)
    ex = (c >> 3) & 0xF
    m = c & 0x7
    val = np.where(ex == 0, m * 2.0 ** -9, (8 + m) * 2.0 ** (ex - 10))
    return s * val


def quantize_rows_fp8_ref(v) -> tuple[np.ndarray, np.ndarray]:
    """Each row of bf16 ``v`` [R,K] -> (e4m3 codes uint8 [R,K], fp32 scale [R])."""
    if isinstance(v, torch.Tensor):
        v = bf16_to_f32(v)
    v = np.asarray(v, dtype=np.float32)
    R, K = v.shape
    amax = np.max(np.abs(v), axis=1) if K else np.zeros(R, np.float32)
    s = (amax / np.float32(E4M3_MAX)).astype(np.float32)   # fp32, correctly rounded
    codes = np.zeros((R, K), dtype=np.uint8)
    nz = amax != 0
    quot = v[nz] / s[nz, None]                               # fp32 quotient, correctly rounded
    codes[nz] = e4m3_encode(e4m3_round(quot.astype(np.float64)))
    return codes, np.where(nz, s, np.float32(0)).astype(np.float32)


def fp8_gemm_ref(cx, cw) -> np.ndarray:
    """Exact acc[m,n] = sum_k x[m,k] * w[n,k] of e4m3 codes (fp64, exact)."""
    return e4m3_decode(cx) @ e4m3_decode(cw).T


def fp32_sum_bound(cx, cw) -> np.ndarray:
    """gamma_K * sum_k |x_k w_k|: the largest error of any fp32 summation order."""
    K = np.asarray(cx).shape[1]
    u = 2.0 ** -24
    gamma = K * u / (1 - K * u)
    return gamma * (np.abs(e4m3_decode(cx)) @ np.abs(e4m3_decode(cw)).T)


def fp8_block_sum_bound(cx, cw) -> np.ndarray:
    """Accumulation error admitted by reading the matrix-core fp8 GEMM as
    blocks of 64 exact products, each block summed with at least 22
    significant bits relative to its largest product, and the block sums
    added in fp32:

      block:  64 terms, each aligned to the largest one's exponent E and
              truncated below 2^(E-21): < 64 * 2^-21 * 2^E <= 2^-15 max|p|
              <= 2^-15 * sum_block |p|;
      blocks: ceil(K/64) fp32 additions, first order
              <= ceil(K/64) * 2^-24 * sum_k |x_k w_k|.

    Returns E_K[m,n] = (2^-15 + ceil(K/64) * 2^-24) * sum_k |x[m,k] w[n,k]|.
    Two bits fewer than fp32's 24 is this reading's allowance for an internal
    adder narrower than fp32; the instruction set does not document the
    block sum's internal precision."""
    K = np.asarray(cx).shape[1]
    rel = 2.0 ** -15 + -(-K // 64) * 2.0 ** -24
    return rel * (np.abs(e4m3_decode(cx)) @ np.abs(e4m3_decode(cw)).T)


def w8a8_fp8_linear_ref(x, w, bias=None) -> dict:
    """The fp8 variant of the whole linear: codes, scales, exact accumulators,
    the fp32 epilogue on them (y32, the same order as the int8 path) and its
    bf16 rounding."""
    cx, s_a = quantize_rows_fp8_ref(x)
    cw, s_w = quantize_rows_fp8_ref(w)
    acc = fp8_gemm_ref(cx, cw)
    y32 = dequant_ref(acc.astype(np.float32), s_a, s_w, bias)
    return dict(cx=cx, s_a=s_a, cw=cw, s_w=s_w, acc=acc, y32=y32, y_bf16=f32_to_bf16_bits(y32))
