"""Thin torch-facing binding of the C ABI in include/w8a8.h.

Argument marshalling only: dtype / device / contiguity checks, output
allocation with torch, and the call on the current HIP stream.  Every
computation runs in libw8a8's HIP kernels.
"""
from __future__ import annotations

import ctypes

import torch

from ._lib import check, lib


def _stream(t: torch.Tensor) -> int:
    return torch.cuda.current_stream(t.device).cuda_stream


def _need(t: torch.Tensor, dtype, ndim: int, name: str) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor (got {t.device})")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype} (got {t.dtype})")
    if t.dim() != ndim:
        raise ValueError(f"{name} must be {ndim}-D (got shape {tuple(t.shape)})")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _quant(fn, x: torch.Tensor, q=None, s=None, name="x", code_dtype=torch.int8):
    _need(x, torch.bfloat16, 2, name)
    R, K = x.shape
    if q is None:
        q = torch.empty((R, K), dtype=code_dtype, device=x.device)
    if s is None:
        s = torch.empty((R,), dtype=torch.float32, device=x.device)
    _need(q, code_dtype, 2, "q")
    _need(s, torch.float32, 1, "scale")
    if tuple(q.shape) != (R, K) or s.shape[0] != R:
        raise ValueError("output shapes do not match the input")
    check(fn(x.data_ptr(), R, K, q.data_ptr(), s.data_ptr(), _stream(x)), fn.__name__)
    return q, s


def quantize_weight(w: torch.Tensor, wq=None, w_scale=None):
    """w bf16 [N,K] -> (wq int8 [N,K], w_scale fp32 [N]), per output channel."""
    return _quant(lib.w8a8_quantize_weight, w, wq, w_scale, "w")


def quantize_act(x: torch.Tensor, xq=None, x_scale=None):
    """x bf16 [M,K] -> (xq int8 [M,K], x_scale fp32 [M]), per token."""
    return _quant(lib.w8a8_quantize_act, x, xq, x_scale, "x")


def dequantize_rows(q: torch.Tensor, scale: torch.Tensor, out=None):
    """q int8 [R,K], scale fp32 [R] -> bf16 [R,K] = bf16(float(q) * scale[row])."""
    _need(q, torch.int8, 2, "q")
    _need(scale, torch.float32, 1, "scale")
    R, K = q.shape
    if scale.shape[0] != R:
        raise ValueError("scale length does not match the rows of q")
    if out is None:
        out = torch.empty((R, K), dtype=torch.bfloat16, device=q.device)
    _need(out, torch.bfloat16, 2, "out")
    if tuple(out.shape) != (R, K):
        raise ValueError("out shape does not match q")
    check(lib.w8a8_dequantize_rows(q.data_ptr(), scale.data_ptr(), R, K, out.data_ptr(), _stream(q)),
          "w8a8_dequantize_rows")
    return out


def quantize_weight_fp8(w: torch.Tensor, wq=None, w_scale=None):
    """w bf16 [N,K] -> (e4m3 codes uint8 [N,K], w_scale fp32 [N]), per output channel."""
    return _quant(lib.w8a8_quantize_weight_fp8, w, wq, w_scale, "w", torch.uint8)


def quantize_act_fp8(x: torch.Tensor, xq=None, x_scale=None):
    """x bf16 [M,K] -> (e4m3 codes uint8 [M,K], x_scale fp32 [M]), per token."""
    return _quant(lib.w8a8_quantize_act_fp8, x, xq, x_scale, "x", torch.uint8)


def _gemm_args(xq, wq, code_dtype=torch.int8):
    _need(xq, code_dtype, 2, "xq")
    _need(wq, code_dtype, 2, "wq")
    M, K = xq.shape
    N, K2 = wq.shape
    if K != K2:
        raise ValueError(f"K mismatch: xq has {K}, wq has {K2}")
    return M, N, K


def linear(xq, x_scale, wq, w_scale, bias=None, y=None, tile: int = -1, gelu: bool = False):
    """Fused W8A8 linear: bf16 y [M,N] = dequant(xq @ wq^T) + bias (through
    GELU before the bf16 rounding when ``gelu``)."""
    M, N, K = _gemm_args(xq, wq)
    _need(x_scale, torch.float32, 1, "x_scale")
    _need(w_scale, torch.float32, 1, "w_scale")
    if x_scale.shape[0] != M or w_scale.shape[0] != N:
        raise ValueError("scale lengths do not match M / N")
    bptr = None
    if bias is not None:
        _need(bias, torch.bfloat16, 1, "bias")
        if bias.shape[0] != N:
            raise ValueError("bias length does not match N")
        bptr = bias.data_ptr()
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _need(y, torch.bfloat16, 2, "y")
    if tuple(y.shape) != (M, N):
        raise ValueError("y shape does not match [M,N]")
    fn = lib.w8a8_linear_gelu_tile if gelu else lib.w8a8_linear_tile
    check(fn(xq.data_ptr(), x_scale.data_ptr(), wq.data_ptr(), w_scale.data_ptr(), bptr, y.data_ptr(),
             M, N, K, tile, _stream(xq)), fn.__name__)
    return y


def select_splitk(M: int, N: int, K: int) -> tuple[int, int]:
    """(K ranges, tile id) the library's split cost model picks for a shape."""
    t = ctypes.c_int(-1)
    c = lib.w8a8_select_splitk(M, N, K, ctypes.byref(t))
    if c < 1:
        raise ValueError("shape outside the GEMM contract")
    return c, t.value


def splitk_workspace_bytes(M: int, N: int, splits: int) -> int:
    return int(lib.w8a8_linear_splitk_workspace(M, N, splits))


def linear_splitk(xq, x_scale, wq, w_scale, bias=None, y=None, splits: int = 0, tile: int = -1,
                  gelu: bool = False, workspace=None):
    """The fused W8A8 linear with K split into `splits` ranges (0: the
    library's choice; 1: no split): the same bits as ``linear``.  The
    workspace (int32 slices of every range) is allocated here unless given
    (a uint8 device tensor of at least splitk_workspace_bytes bytes)."""
    M, N, K = _gemm_args(xq, wq)
    _need(x_scale, torch.float32, 1, "x_scale")
    _need(w_scale, torch.float32, 1, "w_scale")
    if x_scale.shape[0] != M or w_scale.shape[0] != N:
        raise ValueError("scale lengths do not match M / N")
    bptr = None
    if bias is not None:
        _need(bias, torch.bfloat16, 1, "bias")
        if bias.shape[0] != N:
            raise ValueError("bias length does not match N")
        bptr = bias.data_ptr()
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _need(y, torch.bfloat16, 2, "y")
    if tuple(y.shape) != (M, N):
        raise ValueError("y shape does not match [M,N]")
    if splits <= 0:
        splits, auto_tile = select_splitk(M, N, K)
        tile = auto_tile if tile < 0 else tile
    need = splitk_workspace_bytes(M, N, splits)
    if workspace is None:
        workspace = torch.empty((max(need, 16),), dtype=torch.uint8, device=xq.device)
    _need(workspace, torch.uint8, 1, "workspace")
    check(lib.w8a8_linear_splitk(xq.data_ptr(), x_scale.data_ptr(), wq.data_ptr(), w_scale.data_ptr(),
                                 bptr, y.data_ptr(), M, N, K, splits, tile, int(gelu),
                                 workspace.data_ptr(), workspace.numel(), _stream(xq)),
          "w8a8_linear_splitk")
    return y


def gemm_i32(xq, wq, acc=None, tile: int = -1):
    """Raw int32 accumulators acc [M,N] = xq @ wq^T (diagnostic)."""
    M, N, K = _gemm_args(xq, wq)
    if acc is None:
        acc = torch.empty((M, N), dtype=torch.int32, device=xq.device)
    _need(acc, torch.int32, 2, "acc")
    if tuple(acc.shape) != (M, N):
        raise ValueError("acc shape does not match [M,N]")
    check(lib.w8a8_gemm_i32_tile(xq.data_ptr(), wq.data_ptr(), acc.data_ptr(), M, N, K, tile,
                                 _stream(xq)), "w8a8_gemm_i32")
    return acc


def linear_fp8(xq, x_scale, wq, w_scale, bias=None, y=None, tile: int = -1):
    """The fp8 variant: e4m3 codes (uint8) -> bf16 y [M,N] = dequant(xq @ wq^T) + bias."""
    M, N, K = _gemm_args(xq, wq, torch.uint8)
    _need(x_scale, torch.float32, 1, "x_scale")
    _need(w_scale, torch.float32, 1, "w_scale")
    if x_scale.shape[0] != M or w_scale.shape[0] != N:
        raise ValueError("scale lengths do not match M / N")
    bptr = None
    if bias is not None:
        _need(bias, torch.bfloat16, 1, "bias")
        if bias.shape[0] != N:
            raise ValueError("bias length does not match N")
        bptr = bias.data_ptr()
    if y is None:
        y = torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _need(y, torch.bfloat16, 2, "y")
    if tuple(y.shape) != (M, N):
        raise ValueError("y shape does not match [M,N]")
    check(lib.w8a8_linear_fp8_tile(xq.data_ptr(), x_scale.data_ptr(), wq.data_ptr(),
                                   w_scale.data_ptr(), bptr, y.data_ptr(), M, N, K, tile,
                                   _stream(xq)), "w8a8_linear_fp8")
    return y


def gemm_f32_fp8(xq, wq, acc=None, tile: int = -1):
    """fp32 accumulators acc [M,N] = xq @ wq^T of e4m3 codes (diagnostic)."""
    M, N, K = _gemm_args(xq, wq, torch.uint8)
    if acc is None:
        acc = torch.empty((M, N), dtype=torch.float32, device=xq.device)
    _need(acc, torch.float32, 2, "acc")
    if tuple(acc.shape) != (M, N):
        raise ValueError("acc shape does not match [M,N]")
    check(lib.w8a8_gemm_f32_fp8_tile(xq.data_ptr(), wq.data_ptr(), acc.data_ptr(), M, N, K, tile,
                                     _stream(xq)), "w8a8_gemm_f32_fp8")
    return acc


def num_tiles() -> int:
    return lib.w8a8_num_tiles()


def tile_info(tile: int) -> dict:
    v = [ctypes.c_int() for _ in range(4)]
    check(lib.w8a8_tile_info(tile, *[ctypes.byref(t) for t in v]), "w8a8_tile_info")
    return dict(block_m=v[0].value, block_n=v[1].value, block_k=v[2].value, threads=v[3].value)


def select_tile(M: int, N: int, K: int) -> int:
    return lib.w8a8_select_tile(M, N, K)


CEILING_WORKGROUPS = 256
CEILING_MFMAS_PER_ITER = CEILING_WORKGROUPS * 8 * 4 * 6   # workgroups x waves x K steps x MFMAs


def mfma_ceiling(xq: torch.Tensor, wq: torch.Tensor, iters: int, sink=None):
    """Diagnostic: the fused GEMM's K step looped `iters` times on one
    LDS-resident K stage of xq [M,K] / wq [N,K] per workgroup (no memory
    traffic in the loop).  Returns sink int64 [256, 8], each wavefront's
    accumulator sum; the launch does CEILING_MFMAS_PER_ITER * iters int8
    32x32x32 MFMAs (65536 operations each)."""
    _need(xq, torch.int8, 2, "xq")
    _need(wq, torch.int8, 2, "wq")
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K:
        raise ValueError("xq and wq disagree on K")
    if sink is None:
        sink = torch.empty((CEILING_WORKGROUPS, 8), dtype=torch.int64, device=xq.device)
    _need(sink, torch.int64, 2, "sink")
    if tuple(sink.shape) != (CEILING_WORKGROUPS, 8):
        raise ValueError("sink must be int64 [256, 8]")
    check(lib.w8a8_mfma_ceiling(xq.data_ptr(), wq.data_ptr(), M, N, K, iters, sink.data_ptr(),
                                _stream(xq)), "w8a8_mfma_ceiling")
    return sink
