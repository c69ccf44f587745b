"""GPU parity of the K-split fused linear (w8a8_linear_splitk) against the CPU
oracle: the bf16 output must equal bf16(y32) bit for bit (the same gate as
the fused path, since the int32 sum of the K ranges is exact and the epilogue
is the same fp32 expression), with the GELU epilogue within one bf16 ulp of
the fp64 GELU; for several split counts, every tile's main configuration,
ragged M and N, sampled rows of the full 768px shapes, and the workload's
argument errors."""
import numpy as np
import pytest
import torch

import datagen
from oracle import dequant_ref, f32_to_bf16_bits, gelu_ref, int_gemm_ref, quantize_rows_ref
from tests.parity import assert_bf16_close, bf16_bits

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import w8a8_int8_quantized_token_amd as pkg
    return pkg


def _log(msg):
    print(msg, flush=True)


def _oracle(x, W, b, rows):
    ref_wq, ref_ws = quantize_rows_ref(W)
    ref_xq, ref_xs = quantize_rows_ref(x[torch.from_numpy(rows)])
    return dequant_ref(int_gemm_ref(ref_xq, ref_wq), ref_xs, ref_ws, b)


def _check(w, x, W, b, splits, tile=-1, gelu=False, rows=None, label=""):
    M = x.shape[0]
    rows = np.arange(M) if rows is None else rows
    _log(f"[splitk] {label} M,K={tuple(x.shape)} N={W.shape[0]} splits={splits} tile={tile} gelu={gelu}")
    wq, ws = w.quantize_weight(W.to(DEV))
    xq, xs = w.quantize_act(x.to(DEV))
    bd = None if b is None else b.to(DEV)
    y = w.linear_splitk(xq, xs, wq, ws, bd, splits=splits, tile=tile, gelu=gelu)
    torch.cuda.synchronize()
    yb = bf16_bits(y.index_select(0, torch.from_numpy(rows).to(DEV)))
    y32 = _oracle(x, W, b, rows)
    if not gelu:
        assert_bf16_close(yb, y32)
        assert np.array_equal(yb, f32_to_bf16_bits(y32)), "split-K output not bit-identical to bf16(y32)"
    else:
        g64 = gelu_ref(y32)
        assert_bf16_close(yb, g64)
        want = f32_to_bf16_bits(g64.astype(np.float32)).astype(np.int32)
        got = yb.astype(np.int32)
        big = np.abs(g64) >= 1e-30
        assert np.all((((want ^ got) & 0x8000) == 0)[big])
        assert int(np.max(np.abs((got & 0x7FFF) - (want & 0x7FFF))[big], initial=0)) <= 1


@pytest.mark.parametrize("M,N,K", [(1, 8, 64), (33, 136, 192), (257, 264, 3072), (300, 520, 1536),
                                   (129, 256, 12288)])
def test_splitk_ragged(w, M, N, K):
    x = datagen.random_bf16((M, K), seed=M + 17)
    W = datagen.random_bf16((N, K), seed=N + 19, std=0.02)
    b = datagen.random_bf16((N,), seed=K + 23, std=0.01)
    for splits in (1, 2, 3, 4):
        if K % (16 * splits):
            continue
        for tile in (-1, 1, 4, 6):
            _check(w, x, W, b, splits, tile, label="ragged")
    _check(w, x, W, None, 2, label="ragged no bias")
    _check(w, x, W, b, 2, gelu=True, label="ragged gelu")


def test_splitk_many_ranges(w):
    """16 ranges of 768 bytes: every range ends mid-stage of the 128-byte ring."""
    x = datagen.random_bf16((256, 12288), seed=5)
    W = datagen.random_bf16((3072, 12288), seed=6, std=0.02)
    b = datagen.random_bf16((3072,), seed=7, std=0.01)
    _check(w, x, W, b, 16, rows=np.arange(0, 256, 7), label="16 ranges")
    _check(w, x, W, b, 0, rows=np.arange(0, 256, 5), label="automatic")


@pytest.mark.parametrize("li", [0, 1])
def test_splitk_768px_mlp_and_projection(w, li):
    """The 768px DiT shapes (projection 2304x3072->3072; MLP-down
    2304x12288->3072) with every 128-row band sampled, at the split the cost
    model picks and at 3 ranges."""
    wl = datagen.WORKLOADS[1] if li == 0 else datagen.WORKLOADS[2]
    shape = wl.linears[0] if li == 0 else wl.linears[1]
    if shape.act == "gelu_of_prev":
        x = datagen.random_bf16((shape.M, shape.K), seed=wl.seed * 100 + 1)
    else:
        x = datagen.gen_act(shape, wl.seed, 0)
    W, b = datagen.gen_weight(shape, wl.seed, li if li == 0 else 1)
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(0, shape.M, 128) + rng.integers(0, 128, shape.M // 128),
                                     [0, shape.M - 1]]))
    _check(w, x, W, b, 0, rows=rows, label=f"{wl.name} auto")
    _check(w, x, W, b, 3, rows=rows, label=f"{wl.name} 3 ranges")


def test_splitk_errors(w):
    xq = torch.zeros((64, 256), dtype=torch.int8, device=DEV)
    wq = torch.zeros((24, 256), dtype=torch.int8, device=DEV)
    s = torch.ones(64, device=DEV)
    sw = torch.ones(24, device=DEV)
    with pytest.raises(w.W8A8Error):   # K % (16 * splits) != 0
        w.linear_splitk(xq, s, wq, sw, splits=3)
    with pytest.raises(w.W8A8Error):   # N % 8 != 0
        w.linear_splitk(xq, s, wq[:20], sw[:20], splits=2)
    small = torch.empty(16, dtype=torch.uint8, device=DEV)
    with pytest.raises(w.W8A8Error):   # workspace too small
        w.linear_splitk(xq, s, wq, sw, splits=2, workspace=small)
    assert w.splitk_workspace_bytes(64, 24, 2) == 2 * 64 * 24 * 4
    assert w.splitk_workspace_bytes(64, 24, 1) == 0
