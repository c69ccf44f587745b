"""Host-side checks of libw8a8.so that need no GPU: the library loads, it
exports every function include/w8a8.h declares, and argument validation
returns the documented status before anything is launched (the pointers
below are never dereferenced, so fake addresses are safe)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w8a8.h")


@pytest.fixture(scope="module")
def w():
    import w8a8_int8_quantized_token_amd as pkg
    return pkg


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(w8a8_[a-z0-9_]+)\s*\(", text)))


def test_exports_every_declared_symbol(w):
    names = declared_functions()
    assert {"w8a8_quantize_weight", "w8a8_quantize_act", "w8a8_linear", "w8a8_gemm_i32"} <= set(names)
    raw = ctypes.CDLL(w.LIB_PATH)
    for n in names:
        assert hasattr(raw, n), n


def test_status_strings(w):
    for s in range(6):
        assert len(w.status_str(s)) > 0
    assert w.status_str(0) == "ok"
    assert "unknown" in w.status_str(77)


def test_max_k_matches_int32_bound(w):
    assert w.MAX_K == (2 ** 31 - 1) // (127 * 127)
    assert "#define W8A8_MAX_K 133144" in open(HEADER).read()


A = 0x10000   # fake, 16-byte aligned, never dereferenced


@pytest.mark.parametrize("fn", ["w8a8_quantize_weight", "w8a8_quantize_act",
                                "w8a8_quantize_weight_fp8", "w8a8_quantize_act_fp8"])
def test_quantize_validation(w, fn):
    f = getattr(w.lib, fn)
    assert f(None, 4, 64, A, A, None) == 1
    assert f(A, 4, 64, None, A, None) == 1
    assert f(A, 4, 64, A, None, None) == 1
    for R, K in [(-1, 64), (4, 0), (4, 8), (4, 24), (4, 15)]:
        assert f(A, R, K, A, A, None) == 2, (R, K)
    assert f(A + 2, 4, 64, A, A, None) == 3
    assert f(A, 4, 64, A + 8, A, None) == 3
    assert f(A, 4, 64, A, A + 2, None) == 3
    assert f(A, 0, 64, A, A, None) == 0          # empty: no-op, nothing launched
    assert f(None, 0, 64, None, None, None) == 0


@pytest.mark.parametrize("fn", ["w8a8_linear", "w8a8_linear_gelu", "w8a8_linear_fp8"])
def test_linear_validation(w, fn):
    L = getattr(w.lib, fn)
    args = lambda **k: [k.get(n, A) for n in ("xq", "sx", "wq", "sw", "b", "y")] + \
        [k.get("M", 8), k.get("N", 8), k.get("K", 64), None]
    assert L(*args(xq=None)) == 1
    assert L(*args(wq=None)) == 1
    assert L(*args(y=None)) == 1
    assert L(*args(sx=None)) == 1
    assert L(*args(sw=None)) == 1
    for M, N, K in [(-1, 8, 64), (8, 0, 64), (8, 8, 0), (8, 8, 8), (8, 8, 40), (8, 8, 133152)]:
        assert L(*args(M=M, N=N, K=K)) == 2, (M, N, K)
    assert L(*args(xq=A + 4)) == 3
    assert L(*args(wq=A + 1)) == 3
    assert L(*args(y=A + 1)) == 3
    assert L(*args(b=A + 1)) == 3
    assert L(*args(sx=A + 2)) == 3
    assert L(*args(M=0)) == 0
    assert L(*args(M=0, b=None)) == 0
    assert L(*args(M=0, xq=None, sx=None, y=None)) == 0
    assert w.lib.w8a8_linear_tile(*args(M=0)[:-1], 99, None) == 5
    assert w.lib.w8a8_linear_tile(*args(M=0)[:-1], w.num_tiles(), None) == 5


@pytest.mark.parametrize("fn", ["w8a8_gemm_i32", "w8a8_gemm_f32_fp8"])
def test_gemm_raw_validation(w, fn):
    G = getattr(w.lib, fn)
    assert G(None, A, A, 8, 8, 64, None) == 1
    assert G(A, A, None, 8, 8, 64, None) == 1
    assert G(A, A, A, 8, 8, 133144 + 16, None) == 2
    assert G(A, A, A + 2, 8, 8, 64, None) == 3
    assert G(A, A, A, 0, 8, 133136, None) == 0
    assert getattr(w.lib, fn + "_tile")(A, A, A, 0, 8, 64, -7, None) == 0   # negative = automatic
    assert getattr(w.lib, fn + "_tile")(A, A, A, 0, 8, 64, 99, None) == 5


def test_tile_table(w):
    n = w.num_tiles()
    assert n >= 2
    for t in range(n):
        d = w.tile_info(t)
        assert d["block_m"] % 32 == 0 and d["block_n"] % 32 == 0 and d["block_k"] % 32 == 0
        assert d["threads"] % 64 == 0
    assert w.lib.w8a8_tile_info(n, None, None, None, None) == 5
    for M, N, K in [(64, 128, 256), (2304, 3072, 3072), (4096, 9216, 3072), (8192, 3072, 12288), (1, 1, 16)]:
        assert 0 <= w.select_tile(M, N, K) < n


def test_dequantize_validation(w):
    f = w.lib.w8a8_dequantize_rows
    assert f(None, A, 4, 64, A, None) == 1
    assert f(A, None, 4, 64, A, None) == 1
    assert f(A, A, 4, 64, None, None) == 1
    for R, K in [(-1, 64), (4, 0), (4, 8), (4, 24), (4, 15)]:
        assert f(A, A, R, K, A, None) == 2, (R, K)
    assert f(A + 8, A, 4, 64, A, None) == 3
    assert f(A, A + 2, 4, 64, A, None) == 3
    assert f(A, A, 4, 64, A + 8, None) == 3
    assert f(None, None, 0, 64, None, None) == 0   # empty: no-op


def test_plan_choice_on_dit_shapes(w):
    """The cost model picks the plan that was fastest in sweeps over every
    plan on MI355X for these shapes, with the weights cold as inside a model
    (ids: 0 256x256 split ring + 128x256 tail, 4 256x192, 6 256x128,
    8 64x64)."""
    best = {(8192, 9216, 3072): 4, (8192, 3072, 3072): 4, (8192, 12288, 3072): 4,
            (8192, 3072, 12288): 4, (2304, 3072, 3072): 6, (2304, 12288, 3072): 0,
            (2304, 3072, 12288): 6, (4096, 9216, 3072): 4, (64, 128, 256): 8}
    for (M, N, K), plan in best.items():
        assert w.select_tile(M, N, K) == plan, (M, N, K)
