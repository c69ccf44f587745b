"""ctypes loader for libw8a8.so (built in-tree by ``build.py``).

There is no fallback: if the library is missing or does not load, importing
the package raises, so nothing silently runs on another path.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libw8a8.so")

# Status codes of include/w8a8.h
OK, ERR_NULL, ERR_SHAPE, ERR_ALIGN, ERR_LAUNCH, ERR_ARG, ERR_SCRATCH = range(7)
NOALLOC_SCRATCH_BYTES = 32 * 1024 * 1024
MAX_K = 133144


class W8A8Error(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_str(status)} (status {status})")


def _load() -> ctypes.CDLL:
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is not built; run `python w8a8_int8_quantized_token_amd/build.py`")
    lib = ctypes.CDLL(LIB_PATH)
    p, i64, i32, st = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int, ctypes.c_int
    sig = {
        "w8a8_status_str": (ctypes.c_char_p, [st]),
        "w8a8_quantize_weight": (st, [p, i64, i64, p, p, p]),
        "w8a8_quantize_act": (st, [p, i64, i64, p, p, p]),
        "w8a8_dequantize_rows": (st, [p, p, i64, i64, p, p]),
        "w8a8_linear": (st, [p, p, p, p, p, p, i64, i64, i64, p]),
        "w8a8_gemm_i32": (st, [p, p, p, i64, i64, i64, p]),
        "w8a8_num_tiles": (i32, []),
        "w8a8_tile_info": (st, [i32, p, p, p, p]),
        "w8a8_select_tile": (i32, [i64, i64, i64]),
        "w8a8_linear_tile": (st, [p, p, p, p, p, p, i64, i64, i64, i32, p]),
        "w8a8_gemm_i32_tile": (st, [p, p, p, i64, i64, i64, i32, p]),
        "w8a8_linear_gelu": (st, [p, p, p, p, p, p, i64, i64, i64, p]),
        "w8a8_quantize_weight_fp8": (st, [p, i64, i64, p, p, p]),
        "w8a8_quantize_act_fp8": (st, [p, i64, i64, p, p, p]),
        "w8a8_linear_fp8": (st, [p, p, p, p, p, p, i64, i64, i64, p]),
        "w8a8_linear_fp8_tile": (st, [p, p, p, p, p, p, i64, i64, i64, i32, p]),
        "w8a8_gemm_f32_fp8": (st, [p, p, p, i64, i64, i64, p]),
        "w8a8_gemm_f32_fp8_tile": (st, [p, p, p, i64, i64, i64, i32, p]),
        "w8a8_linear_gelu_tile": (st, [p, p, p, p, p, p, i64, i64, i64, i32, p]),
        "w8a8_mfma_ceiling": (st, [p, p, i64, i64, i64, i64, p, p]),
        "w8a8_select_splitk": (i32, [i64, i64, i64, p]),
        "w8a8_linear_splitk_workspace": (ctypes.c_size_t, [i64, i64, i32]),
        "w8a8_linear_splitk": (st, [p, p, p, p, p, p, i64, i64, i64, i32, i32, i32, p, ctypes.c_size_t, p]),
        "w8a8_linear_splitk_noalloc": (st, [p, p, p, p, p, p, i64, i64, i64, i32, i32, i32, p]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


def status_str(status: int) -> str:
    return lib.w8a8_status_str(status).decode()


def check(status: int, where: str) -> None:
    if status != OK:
        raise W8A8Error(status, where)
