"""GPU parity of the fp8 (e4m3) variant against the oracle: e4m3 codes and
fp32 scales bit for bit; fp32 accumulators within the matrix-core bound of
the exact sum (oracle.fp8.fp8_mfma_bound); the bf16 output bit for bit equal to the oracle's epilogue
applied to the GPU's own accumulators, and within the accumulation bound carried through
the dequantization (plus one bf16 ulp) of the epilogue applied to the exact
ones."""
import numpy as np
import pytest
import torch

import datagen
from oracle import (dequant_ref, f32_to_bf16_bits, fp8_gemm_ref, fp8_mfma_bound,
                    quantize_rows_fp8_ref)
from tests.parity import COS_MIN, bf16_bits, bf16_metrics, bits_to_f32

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


def test_fp8_quantizer_bit_exact(w):
    rng = np.random.default_rng(12)
    rows = [rng.standard_normal(1024) * 3,
            rng.standard_t(3, 1024) * 0.01,
            np.zeros(1024),
            np.full(1024, 2.0 ** -130),                           # subnormal-range inputs
            np.linspace(-448, 448, 1024) * 2.0 ** -20,             # amax = 448 * 2^-20: exact codes
            (rng.integers(-127, 128, 1024) / 127.0) * 1e30,
            np.where(np.arange(1024) % 3 == 0, -0.0, rng.standard_normal(1024))]   # signed zeros
    x = torch.from_numpy(np.stack(rows).astype(np.float32)).to(torch.bfloat16)
    for K in (16, 1024):
        xs = x[:, :K].contiguous()
        q, s = w.quantize_act_fp8(xs.to(DEV))
        qw, sw = w.quantize_weight_fp8(xs.to(DEV))
        torch.cuda.synchronize()
        ref_q, ref_s = quantize_rows_fp8_ref(xs)
        assert np.array_equal(q.cpu().numpy(), ref_q)
        assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
        assert np.array_equal(qw.cpu().numpy(), ref_q)


@pytest.mark.parametrize("wl_index,rows", [(1, 512), (4, 384)])
def test_fp8_quantizer_workloads(w, wl_index, rows):
    wl = datagen.WORKLOADS[wl_index]
    shape = wl.linears[-1]
    x = datagen.gen_act(shape, wl.seed, len(wl.linears) - 1, rows=np.arange(rows))
    q, s = w.quantize_act_fp8(x.to(DEV))
    torch.cuda.synchronize()
    ref_q, ref_s = quantize_rows_fp8_ref(x)
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def _check_y(yb, exact, cx, cw, sx, sw, b):
    """bf16 output against the epilogue on the exact accumulators: the
    accumulation bound carried through the (linear) dequantization, plus one
    bf16 ulp and the fp32 epilogue roundings; cosine >= 0.9999."""
    y = bits_to_f32(yb).astype(np.float64)
    bb = np.zeros(exact.shape[1]) if b is None else bits_to_f32(b.view(torch.int16).numpy().view(np.uint16)).astype(np.float64)
    yref = dequant_ref(exact.astype(np.float32), sx, sw, b).astype(np.float64)
    scale = sx.astype(np.float64)[:, None] * sw.astype(np.float64)[None, :]
    tol = (fp8_mfma_bound(cx, cw) * scale * (1 + 1e-6) + 2.0 ** -8 * np.abs(yref)
           + 4 * 2.0 ** -24 * (np.abs(exact) * scale + np.abs(bb)[None, :]))
    assert np.all(np.abs(y - yref) <= tol), float(np.max(np.abs(y - yref) / tol))
    m = bf16_metrics(yb, yref)
    assert m["finite"] and m["cos"] >= COS_MIN, m
    return m


def _check_acc(acc_gpu, cx, cw):
    exact = fp8_gemm_ref(cx, cw)
    bound = fp8_mfma_bound(cx, cw)
    err = np.abs(acc_gpu.astype(np.float64) - exact)
    assert np.all(err <= bound), float((err - bound).max())
    return exact


@pytest.mark.parametrize("M,N,K", [(2, 3, 16), (65, 64, 1040), (257, 260, 3072), (129, 255, 12288)])
def test_fp8_gemm_all_tiles(w, M, N, K):
    x = datagen.random_bf16((M, K), seed=M + 5)
    W = datagen.random_bf16((N, K), seed=N + 9, std=0.02)
    b = datagen.random_bf16((N,), seed=K + 3, std=0.01)
    cx, sx = w.quantize_act_fp8(x.to(DEV))
    cw, sw = w.quantize_weight_fp8(W.to(DEV))
    ref_cx, ref_sx = quantize_rows_fp8_ref(x)
    ref_cw, ref_sw = quantize_rows_fp8_ref(W)
    for tile in range(w.num_tiles()):
        _log(f"[fp8] gemm M={M} N={N} K={K} tile={tile}")
        acc = w.gemm_f32_fp8(cx, cw, tile=tile)
        y = w.linear_fp8(cx, sx, cw, sw, b.to(DEV), tile=tile)
        torch.cuda.synchronize()
        assert np.array_equal(cx.cpu().numpy(), ref_cx) and np.array_equal(cw.cpu().numpy(), ref_cw)
        a = acc.cpu().numpy()
        exact = _check_acc(a, ref_cx, ref_cw)
        yb = bf16_bits(y)
        # the epilogue is deterministic given the accumulators
        assert np.array_equal(yb, f32_to_bf16_bits(dequant_ref(a, ref_sx, ref_sw, b)))
        _check_y(yb, exact, ref_cx, ref_cw, ref_sx, ref_sw, b)


def test_fp8_linear_full_size_sampled(w):
    wl = datagen.WORKLOADS[4]
    shape = wl.linears[0]   # QKV 8192 x 3072 -> 9216
    _log("[fp8] QKV full size")
    x = datagen.gen_act(shape, wl.seed, 0)
    W, b = datagen.gen_weight(shape, wl.seed, 0)
    cx, sx = w.quantize_act_fp8(x.to(DEV))
    cw, sw = w.quantize_weight_fp8(W.to(DEV))
    y = w.linear_fp8(cx, sx, cw, sw, b.to(DEV))
    acc = w.gemm_f32_fp8(cx, cw)
    torch.cuda.synchronize()
    rows = np.unique(np.concatenate([[0, 255, 256, 4095, 8191], np.random.default_rng(7).choice(8192, 40, replace=False)]))
    ref_cx, ref_sx = quantize_rows_fp8_ref(x[torch.from_numpy(rows)])
    ref_cw, ref_sw = quantize_rows_fp8_ref(W)
    ridx = torch.from_numpy(rows).to(DEV)
    assert np.array_equal(cx.index_select(0, ridx).cpu().numpy(), ref_cx)
    assert np.array_equal(cw.cpu().numpy(), ref_cw)
    a = acc.index_select(0, ridx).cpu().numpy()
    exact = _check_acc(a, ref_cx, ref_cw)
    yb = bf16_bits(y.index_select(0, ridx))
    assert np.array_equal(yb, f32_to_bf16_bits(dequant_ref(a, ref_sx, ref_sw, b)))
    m = _check_y(yb, exact, ref_cx, ref_cw, ref_sx, ref_sw, b)
    _log(f"[fp8] QKV ok cos={m['cos']:.7f} rel={m['rel']:.2e}")
