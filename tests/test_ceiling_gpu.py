"""GPU check of the matrix-core ceiling diagnostic (w8a8_mfma_ceiling): the
sums of each workgroup's int32 accumulators equal the closed form
iters * sum_k (sum_m x[m0+m, k0+k]) * (sum_n w[n0+n, k0+k]) over the
workgroup's 256 rows of xq, 192 rows of wq and 128-byte K stage, computed
exactly here in int64 from codes drawn on the host."""
import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import w8a8_int8_quantized_token_amd as pkg
    return pkg


def expected_sums(x, wt, iters):
    M, K = x.shape
    N = wt.shape[0]
    tm, tn, tk = M // 256, N // 192, K // 128
    out = np.zeros(256, dtype=np.int64)
    for g in range(256):
        m0, n0, k0 = (g % tm) * 256, ((g // tm) % tn) * 192, (g % tk) * 128
        xs = x[m0:m0 + 256, k0:k0 + 128].astype(np.int64).sum(axis=0)
        ws = wt[n0:n0 + 192, k0:k0 + 128].astype(np.int64).sum(axis=0)
        out[g] = iters * int((xs * ws).sum())
    return out


@pytest.mark.parametrize("M,N,K,iters", [(256, 192, 128, 1), (512, 384, 384, 3), (1000, 600, 272, 7)])
def test_ceiling_accumulator_sums(w, M, N, K, iters):
    rng = np.random.default_rng(M + N + K)
    x = rng.integers(-127, 128, (M, K), dtype=np.int8)
    wt = rng.integers(-127, 128, (N, K), dtype=np.int8)
    sink = w.mfma_ceiling(torch.from_numpy(x).to(DEV), torch.from_numpy(wt).to(DEV), iters)
    torch.cuda.synchronize()
    got = sink.cpu().numpy().sum(axis=1)
    assert np.array_equal(got, expected_sums(x, wt, iters))


def test_ceiling_rejects_small_shapes(w):
    x = torch.zeros((256, 128), dtype=torch.int8, device=DEV)
    with pytest.raises(w.W8A8Error):
        w.mfma_ceiling(x[:255], torch.zeros((192, 128), dtype=torch.int8, device=DEV), 1)
    with pytest.raises(w.W8A8Error):
        w.mfma_ceiling(x, torch.zeros((191, 128), dtype=torch.int8, device=DEV), 1)
    with pytest.raises(w.W8A8Error):
        w.mfma_ceiling(x, torch.zeros((192, 128), dtype=torch.int8, device=DEV), 0)
