"""GPU parity of the row quantizers (int8 per token / per channel, and the
e4m3 variant) across every row-length specialization of the kernel: rows
held in registers for 1 to 24 chunks per lane (K up to 12288), and the
two-pass kernel beyond (K = 12304 and 65536).  Codes and fp32 scales are
compared bit for bit with the oracle."""
import numpy as np
import pytest
import torch

from oracle import quantize_rows_fp8_ref, quantize_rows_ref

pytestmark = pytest.mark.gpu

DEV = "cuda:0"

# 16-byte chunks per lane = ceil(K / 8 / 64); one K per specialization, ragged ones included
K_VALUES = [16, 512, 528, 1024, 2048, 3072, 4096, 6144, 8192, 12288, 12304, 65536]


@pytest.fixture(scope="module")
def w():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import w8a8_int8_quantized_token_amd as pkg
    return pkg


def rows_for(K: int, seed: int) -> torch.Tensor:
    rng = np.random.default_rng(seed)
    rows = [rng.standard_normal(K),
            rng.standard_t(3, K) * 0.02,
            np.zeros(K),
            np.full(K, 2.0 ** -130),                            # subnormal-range inputs
            np.where(np.arange(K) == K - 1, 300.0, rng.standard_normal(K) * 1e-3),   # max in the last chunk
            np.where(np.arange(K) == 0, -7.0, rng.uniform(-1, 1, K)),                # max first, negative
            (rng.integers(-127, 128, K) / 127.0) * 2.0 ** 20]
    return torch.from_numpy(np.stack(rows).astype(np.float32)).to(torch.bfloat16)


@pytest.mark.parametrize("K", K_VALUES)
def test_int8_quantizer_every_row_length(w, K):
    x = rows_for(K, K)
    q, s = w.quantize_act(x.to(DEV))
    qw, sw = w.quantize_weight(x.to(DEV))
    torch.cuda.synchronize()
    ref_q, ref_s = quantize_rows_ref(x)
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
    assert np.array_equal(qw.cpu().numpy(), ref_q)
    assert np.array_equal(sw.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


@pytest.mark.parametrize("K", K_VALUES)
def test_fp8_quantizer_every_row_length(w, K):
    x = rows_for(K, K + 1)
    q, s = w.quantize_act_fp8(x.to(DEV))
    torch.cuda.synchronize()
    ref_q, ref_s = quantize_rows_fp8_ref(x)
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))
