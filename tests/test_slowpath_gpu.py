"""GPU checks of the dequantize-to-bf16 path (the production path that the
abstract of arXiv 2606.14598 replaces, kept as a measured comparator):
the dequantization kernel bit for bit against the oracle, and the whole path
(quantize -> dequantize -> bf16 GEMM) within the bf16 tolerance."""
import numpy as np
import pytest
import torch

import datagen
from oracle import dequant_bf16_linear_ref, dequant_rows_ref, quantize_rows_ref
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


@pytest.mark.parametrize("R,K", [(1, 16), (37, 272), (300, 3072), (64, 12288)])
def test_dequantize_rows_bit_exact(w, R, K):
    _log(f"[slowpath] dequantize R={R} K={K}")
    rng = np.random.default_rng(R * 7 + K)
    q = rng.integers(-127, 128, size=(R, K), dtype=np.int8)
    q[0, :3] = [127, -127, 0]
    s = (rng.random(R).astype(np.float32) * np.float32(0.05))
    special = np.array([0.0, 2.0 ** -149, 2.0 ** -126, 1.0 + 2.0 ** -8, 3.0e30], dtype=np.float32)
    s[:min(R, special.size)] = special[:min(R, special.size)]
    out = w.dequantize_rows(torch.from_numpy(q).to(DEV), torch.from_numpy(s).to(DEV))
    torch.cuda.synchronize()
    assert np.array_equal(bf16_bits(out), dequant_rows_ref(q, s))


def test_dequantize_empty_and_errors(w):
    q = torch.empty((0, 64), dtype=torch.int8, device=DEV)
    s = torch.empty((0,), dtype=torch.float32, device=DEV)
    assert w.dequantize_rows(q, s).shape == (0, 64)
    with pytest.raises(w.W8A8Error):
        w.dequantize_rows(torch.zeros((4, 24), dtype=torch.int8, device=DEV),
                          torch.ones(4, dtype=torch.float32, device=DEV))


@pytest.mark.parametrize("wl_index,rows", [(0, None), (3, 512)])
def test_dequant_bf16_linear(w, wl_index, rows):
    wl = datagen.WORKLOADS[wl_index]
    shape = wl.linears[0]
    _log(f"[slowpath] linear {wl.name} rows={rows}")
    x = datagen.gen_act(shape, wl.seed, rows=None if rows is None else np.arange(rows))
    W, b = datagen.gen_weight(shape, wl.seed)
    wq, ws = w.quantize_weight(W.to(DEV))
    y = w.dequant_bf16_linear(x.to(DEV), wq, ws, b.to(DEV))
    torch.cuda.synchronize()
    ref_wq, ref_ws = quantize_rows_ref(W)
    assert np.array_equal(wq.cpu().numpy(), ref_wq)
    ref = dequant_bf16_linear_ref(x, ref_wq, ref_ws, b)
    m = assert_bf16_close(bf16_bits(y), ref["y64"])
    _log(f"[slowpath] linear ok cos={m['cos']:.7f} rel={m['rel']:.2e}")
