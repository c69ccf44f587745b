"""GPU parity: libw8a8 (through its C ABI) against the CPU oracle.

int8 codes, fp32 scales and int32 accumulators must match bit for bit; the
bf16 output must meet the tolerance (max rel err <= 1e-2 with a floor,
cosine >= 0.9999, no NaN/Inf) and, because the epilogue evaluates the same
fp32 expression in the same order, is also expected to match bit for bit.
Full-size workloads compare, for the GEMM, token rows (every column) that
include one row of every 128-row band and the band edges, so every output
tile of every plan (tiles are at most 256 rows tall) of the persistent,
XCD-rotated walk is checked; the quantizers are compared on every element.
"""
import numpy as np
import pytest
import torch

import datagen
from oracle import (bf16_to_f32, dequant_ref, dequant_ref64, f32_to_bf16_bits, gelu_ref,
                    int_gemm_ref, quantize_rows_ref)
from tests.parity import assert_bf16_close, bf16_bits

pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def w():
    if not torch.cuda.is_available():
        pytest.fail("GPU tests need a visible GPU")
    import w8a8_int8_quantized_token_amd as pkg   # raises if libw8a8.so is missing
    return pkg


def _log(msg):
    print(msg, flush=True)


def sample_rows(M: int, n: int, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    edge = [0, 1, 31, 32, 127, 128, 255, 256, M // 2, M - 257, M - 256, M - 2, M - 1]
    rows = np.unique(np.concatenate([[r for r in edge if 0 <= r < M], rng.choice(M, min(n, M), replace=False)]))
    return rows.astype(np.int64)


def band_rows(M: int, seed: int, band: int = 128) -> np.ndarray:
    """One random row in every `band`-row band of [0, M) plus the first and
    last row of the first, a middle and the last band: every output tile
    whose height divides into `band`-row bands gets at least one row."""
    rng = np.random.default_rng(seed)
    starts = np.arange(0, M, band)
    picks = starts + rng.integers(0, band, starts.size)
    picks = np.minimum(picks, M - 1)
    mid = (M // 2) // band * band
    edge = [0, min(band, M) - 1, mid, min(mid + band, M) - 1, starts[-1], M - 1]
    return np.unique(np.concatenate([picks, edge])).astype(np.int64)


def check_quant_chunked(q, s, x_cpu, rows_per_chunk: int):
    """Every element of q, s against the oracle, a chunk of rows at a time."""
    M = x_cpu.shape[0]
    for r0 in range(0, M, rows_per_chunk):
        r1 = min(M, r0 + rows_per_chunk)
        rq, rs = quantize_rows_ref(x_cpu[r0:r1])
        check_quant(q[r0:r1], s[r0:r1], rq, rs)


def gpu_quant(w, t_cpu, weight=False):
    t = t_cpu.to(DEV)
    q, s = (w.quantize_weight if weight else w.quantize_act)(t)
    return t, q, s


def check_quant(q, s, ref_q, ref_s):
    assert np.array_equal(q.cpu().numpy(), ref_q)
    assert np.array_equal(s.cpu().numpy().view(np.uint32), ref_s.view(np.uint32))


def run_linear_check(w, x_cpu, W_cpu, b_cpu, rows=None, tile=-1, label=""):
    """Quantize + GEMM + epilogue on the GPU; compare everything with the oracle."""
    _log(f"[parity] {label} M,K={tuple(x_cpu.shape)} N={W_cpu.shape[0]} tile={tile}")
    M = x_cpu.shape[0]
    rows = np.arange(M) if rows is None else rows
    wd, wq, ws = gpu_quant(w, W_cpu, weight=True)
    xd, xq, xs = gpu_quant(w, x_cpu)
    bd = None if b_cpu is None else b_cpu.to(DEV)
    y = w.linear(xq, xs, wq, ws, bd, tile=tile)
    acc = w.gemm_i32(xq, wq, tile=tile)
    torch.cuda.synchronize()
    ref_wq, ref_ws = quantize_rows_ref(W_cpu)
    check_quant(wq, ws, ref_wq, ref_ws)
    ref_xq, ref_xs = quantize_rows_ref(x_cpu[torch.from_numpy(rows)])
    ridx = torch.from_numpy(rows).to(DEV)
    check_quant(xq.index_select(0, ridx), xs.index_select(0, ridx), ref_xq, ref_xs)
    ref_acc = int_gemm_ref(ref_xq, ref_wq)
    assert np.array_equal(acc.index_select(0, ridx).cpu().numpy(), ref_acc)
    y32 = dequant_ref(ref_acc, ref_xs, ref_ws, b_cpu)
    y64 = dequant_ref64(ref_acc, ref_xs, ref_ws, b_cpu)
    yb = bf16_bits(y.index_select(0, ridx))
    m = assert_bf16_close(yb, y32, y64)
    assert np.array_equal(yb, f32_to_bf16_bits(y32)), "bf16 output not bit-identical to bf16(y32)"
    _log(f"[parity] {label} ok cos={m['cos']:.7f} rel={m['rel']:.2e}")
    return y, xq, wq


# ---------------------------------------------------------------- workloads
@pytest.mark.parametrize("idx", [0, 1, 3, 4])
def test_workload(w, idx):
    wl = datagen.WORKLOADS[idx]
    for li, shape in enumerate(wl.linears):
        x = datagen.gen_act(shape, wl.seed, li)
        W, b = datagen.gen_weight(shape, wl.seed, li)
        rows = None if shape.M <= 256 else band_rows(shape.M, 1000 + li)
        # full quantizer parity on every element
        xd, xq, xs = gpu_quant(w, x)
        torch.cuda.synchronize()
        check_quant_chunked(xq, xs, x, max(1, (16 << 20) // shape.K))
        del xd, xq, xs
        run_linear_check(w, x, W, b, rows, label=f"{wl.name}/{shape.name}")


def run_gelu_check(w, x_cpu, W_cpu, b_cpu, rows=None, tile=-1, label=""):
    """Quantize + GEMM + dequant + GELU epilogue on the GPU against the oracle's
    fp32 dequant followed by the fp64 GELU: bf16 tolerance, and no element more
    than one bf16 ulp from bf16(gelu(y32))."""
    _log(f"[parity] gelu {label} M,K={tuple(x_cpu.shape)} N={W_cpu.shape[0]} tile={tile}")
    M = x_cpu.shape[0]
    rows = np.arange(M) if rows is None else rows
    _, wq, ws = gpu_quant(w, W_cpu, weight=True)
    _, xq, xs = gpu_quant(w, x_cpu)
    bd = None if b_cpu is None else b_cpu.to(DEV)
    h = w.linear(xq, xs, wq, ws, bd, tile=tile, gelu=True)
    torch.cuda.synchronize()
    ref_wq, ref_ws = quantize_rows_ref(W_cpu)
    ref_xq, ref_xs = quantize_rows_ref(x_cpu[torch.from_numpy(rows)])
    y32 = dequant_ref(int_gemm_ref(ref_xq, ref_wq), ref_xs, ref_ws, b_cpu)
    g64 = gelu_ref(y32)
    hb = bf16_bits(h.index_select(0, torch.from_numpy(rows).to(DEV)))
    m = assert_bf16_close(hb, g64)
    # one bf16 ulp at most from the correctly rounded fp64 GELU
    want = f32_to_bf16_bits(g64.astype(np.float32)).astype(np.int32)
    got = hb.astype(np.int32)
    big = np.abs(g64) >= 1e-30   # below that the fp32 exp underflows: compared by tolerance only
    assert np.all((((want ^ got) & 0x8000) == 0)[big])
    assert int(np.max(np.abs((got & 0x7FFF) - (want & 0x7FFF))[big], initial=0)) <= 1
    _log(f"[parity] gelu {label} ok cos={m['cos']:.7f} rel={m['rel']:.2e}")
    return h


def test_mlp_pair_stagewise(w):
    """Up-projection with the GELU epilogue, then the down-projection on the
    GPU's own GELU output, re-quantized per token (stage-wise parity)."""
    wl = datagen.WORKLOADS[2]
    up, down = wl.linears
    x = datagen.gen_act(up, wl.seed, 0)
    Wu, bu = datagen.gen_weight(up, wl.seed, 0)
    Wd, bd = datagen.gen_weight(down, wl.seed, 1)
    rows = sample_rows(up.M, 48, 2000)
    h = run_gelu_check(w, x, Wu, bu, rows, label="mlp_up")
    run_linear_check(w, h.cpu(), Wd, bd, rows, label="mlp_down")


@pytest.mark.parametrize("M,N,K", [(2, 3, 16), (65, 64, 1040), (257, 260, 3072), (129, 255, 12288)])
def test_gelu_epilogue_ragged(w, M, N, K):
    x = datagen.random_bf16((M, K), seed=M + 70)
    W = datagen.random_bf16((N, K), seed=N + 110, std=0.02)
    b = datagen.random_bf16((N,), seed=K + 1, std=0.5)
    for tile in range(w.num_tiles()):
        run_gelu_check(w, x, W, b, tile=tile, label=f"ragged tile{tile}")


# ---------------------------------------------------------------- edge cases
@pytest.mark.parametrize("M,N,K", [(1, 128, 256), (2, 3, 16), (31, 100, 272), (33, 129, 48),
                                   (65, 64, 1040), (257, 260, 3072), (1000, 1, 128),
                                   (300, 4098, 64), (129, 255, 12288)])
def test_ragged_shapes(w, M, N, K):
    x = datagen.random_bf16((M, K), seed=M + 7)
    W = datagen.random_bf16((N, K), seed=N + 11, std=0.02)
    b = datagen.random_bf16((N,), seed=K, std=0.01)
    for tile in range(w.num_tiles()):
        run_linear_check(w, x, W, b, tile=tile, label=f"ragged tile{tile}")


@pytest.mark.parametrize("M,N,K", [(4096, 4352, 256), (4100, 4344, 272)])
def test_main_plus_tail_split(w, M, N, K):
    """Shapes whose 256x256 tiles overflow a whole wave of the 256 CUs by one
    column: the leading columns run as 256x256 tiles, the rest as a second
    launch of 128x256 tiles writing into the same output rows."""
    x = datagen.random_bf16((M, K), seed=M)
    W = datagen.random_bf16((N, K), seed=N, std=0.02)
    b = datagen.random_bf16((N,), seed=K, std=0.01)
    rows = sample_rows(M, 48, 7)
    for tile in range(w.num_tiles()):
        run_linear_check(w, x, W, b, rows, tile=tile, label=f"split tile{tile}")


@pytest.mark.parametrize("M,N,K", [(16384, 576, 256), (8192, 2304, 320), (8192, 768, 272)])
def test_rotated_column_walk(w, M, N, K):
    """Grids in which every XCD owns whole groups of tile rows, so the
    per-XCD rotation of the column walk applies (with 1 and 2 groups per XCD
    and column counts that the rotation wraps around): every output tile must
    still be computed exactly once."""
    x = datagen.random_bf16((M, K), seed=M + N)
    W = datagen.random_bf16((N, K), seed=N + 3, std=0.02)
    b = datagen.random_bf16((N,), seed=K + 5, std=0.01)
    rows = sample_rows(M, 40, 11)
    for tile in range(w.num_tiles()):
        run_linear_check(w, x, W, b, rows, tile=tile, label=f"rotated walk tile{tile}")


@pytest.mark.parametrize("M,N,K,with_bias", [(8192, 3072, 256, False), (8192, 3072, 1040, True)])
def test_per_tile_scalars(w, M, N, K, with_bias):
    """Several tiles per workgroup with a short K loop (one or two blocks of
    six stages), with and without bias: each tile's dequant scalars are
    requested during its own last stages, so a tile must never see its
    neighbour's scales or bias."""
    x = datagen.random_bf16((M, K), seed=K + 17)
    W = datagen.random_bf16((N, K), seed=K + 19, std=0.02)
    b = datagen.random_bf16((N,), seed=K + 23, std=0.01) if with_bias else None
    rows = sample_rows(M, 40, K)
    for tile in range(w.num_tiles()):
        run_linear_check(w, x, W, b, rows, tile=tile, label=f"per-tile scalars tile{tile}")


def _pattern_rows(rows: np.ndarray, K: int) -> torch.Tensor:
    """x[m, k] = ((7m + 13k) mod 251 - 125) / 64, exact in bf16, for the given rows (CPU)."""
    m = torch.from_numpy(rows.astype(np.int64))[:, None]
    k = torch.arange(K, dtype=torch.int64)[None, :]
    return (((7 * m + 13 * k) % 251 - 125).to(torch.float32) / 64).to(torch.bfloat16)


def test_operands_beyond_4gib(w):
    """Activation codes of more than 2^32 bytes (M = 1,050,001 tokens at
    K = 4096): rows on both sides of the 4 GiB boundary and the ragged last
    row match the oracle, so no row offset wraps at 32 bits."""
    M, K, N = 1_050_001, 4096, 80
    x = torch.empty((M, K), dtype=torch.bfloat16, device=DEV)
    kk = (13 * torch.arange(K, device=DEV, dtype=torch.int32)) % 251
    for r0 in range(0, M, 1 << 16):
        r1 = min(M, r0 + (1 << 16))
        mm = (7 * torch.arange(r0, r1, device=DEV, dtype=torch.int32)) % 251
        x[r0:r1] = (((mm[:, None] + kk[None, :]) % 251 - 125).to(torch.float32) / 64).to(torch.bfloat16)
    W = datagen.random_bf16((N, K), seed=4096 + N, std=0.02)
    b = datagen.random_bf16((N,), seed=4097, std=0.01)
    xq, xs = w.quantize_act(x)
    del x
    wq, ws = w.quantize_weight(W.to(DEV))
    y = w.linear(xq, xs, wq, ws, b.to(DEV))
    acc = w.gemm_i32(xq, wq)
    torch.cuda.synchronize()
    edge = (1 << 32) // K   # first row past 4 GiB of codes
    rows = np.unique(np.array([0, 1, 255, 256, edge - 257, edge - 2, edge - 1, edge, edge + 1,
                               edge + 255, M - 257, M - 2, M - 1]))
    rows = np.concatenate([rows, np.random.default_rng(7).choice(M, 24, replace=False)])
    rows = np.unique(rows)
    ref_xq, ref_xs = quantize_rows_ref(_pattern_rows(rows, K))
    ref_wq, ref_ws = quantize_rows_ref(W)
    ridx = torch.from_numpy(rows).to(DEV)
    check_quant(xq.index_select(0, ridx), xs.index_select(0, ridx), ref_xq, ref_xs)
    check_quant(wq, ws, ref_wq, ref_ws)
    ref_acc = int_gemm_ref(ref_xq, ref_wq)
    assert np.array_equal(acc.index_select(0, ridx).cpu().numpy(), ref_acc)
    y32 = dequant_ref(ref_acc, ref_xs, ref_ws, b)
    yb = bf16_bits(y.index_select(0, ridx))
    assert np.array_equal(yb, f32_to_bf16_bits(y32))
    del xq, acc, y
    torch.cuda.empty_cache()


def test_special_rows(w):
    """Zero rows give exactly the bias; huge, tiny (subnormal-scale) and
    single-spike rows quantize bit-exactly."""
    M, N, K = 40, 96, 512
    xf = datagen.random_bf16((M, K), seed=3).float()
    xf[0] = 0
    xf[7] = 0
    xf[5] *= 1e30
    xf[6] *= 1e-36                                     # scale below 2^-100
    xf[8] = 0
    xf[8, 17] = -3.0e-39                               # one subnormal value
    xf[9] = 0
    xf[9, 100] = 2.0 ** -133                           # the smallest bf16 subnormal
    xf[10] *= 1e-20
    xf[11] = torch.where(torch.arange(K) % 2 == 0, 1.0, -1.0)
    xf[12, 3] = 1e4                                    # single outlier in a normal row
    x = xf.to(torch.bfloat16)
    W = datagen.random_bf16((N, K), seed=4, std=0.02)
    b = datagen.random_bf16((N,), seed=5, std=0.01)
    y, xq, _ = run_linear_check(w, x, W, b, label="special rows")
    yb = bf16_bits(y)
    bb = b.view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(yb[0], bb) and np.array_equal(yb[7], bb)
    run_linear_check(w, x, W, None, label="special rows, no bias")


def test_extreme_codes_closed_form(w):
    """All +-127 codes at K=12288: acc = +-16129*K exactly (no int32 overflow)."""
    M, N, K = 64, 64, 12288
    xq = torch.full((M, K), 127, dtype=torch.int8, device=DEV)
    xq[1::2] = -127
    wq = torch.full((N, K), 127, dtype=torch.int8, device=DEV)
    wq[::3] = -127
    acc = w.gemm_i32(xq, wq).cpu().numpy().astype(np.int64)
    sign = np.where(np.arange(M)[:, None] % 2 == 1, -1, 1) * np.where(np.arange(N)[None, :] % 3 == 0, -1, 1)
    assert np.array_equal(acc, sign * 16129 * K)


def test_largest_k_closed_form_every_plan(w):
    """At the largest K the boundary accepts that is a multiple of 16
    (133136; the int32 bound is 133144), all +-127 codes give
    acc = +-16129*K = +-2147350544 exactly on every tile plan: the int32
    accumulators come within 0.01% of overflow and do not wrap."""
    K = (w.MAX_K // 16) * 16
    M, N = 40, 72
    xq = torch.full((M, K), 127, dtype=torch.int8, device=DEV)
    xq[1::2] = -127
    wq = torch.full((N, K), 127, dtype=torch.int8, device=DEV)
    wq[::3] = -127
    sign = np.where(np.arange(M)[:, None] % 2 == 1, -1, 1) * np.where(np.arange(N)[None, :] % 3 == 0, -1, 1)
    for tile in range(w.num_tiles()):
        acc = w.gemm_i32(xq, wq, tile=tile).cpu().numpy().astype(np.int64)
        assert np.array_equal(acc, sign * 16129 * K), tile


def test_unit_scales_zero_bias_give_bf16_of_acc(w):
    M, N, K = 96, 80, 256
    xq = torch.from_numpy(datagen.random_int8((M, K), 1)).to(DEV)
    wq = torch.from_numpy(datagen.random_int8((N, K), 2)).to(DEV)
    ones_m = torch.ones(M, dtype=torch.float32, device=DEV)
    ones_n = torch.ones(N, dtype=torch.float32, device=DEV)
    y = w.linear(xq, ones_m, wq, ones_n, None)
    acc = int_gemm_ref(xq.cpu().numpy(), wq.cpu().numpy())
    assert np.array_equal(bf16_bits(y), f32_to_bf16_bits(acc.astype(np.float32)))


def test_tiles_bit_identical(w):
    M, N, K = 700, 520, 1536
    xq = torch.from_numpy(datagen.random_int8((M, K), 5)).to(DEV)
    wq = torch.from_numpy(datagen.random_int8((N, K), 6)).to(DEV)
    sx = torch.rand(M, device=DEV) * 0.01
    sw = torch.rand(N, device=DEV) * 0.01
    b = (torch.randn(N, device=DEV) * 0.01).to(torch.bfloat16)
    outs = [bf16_bits(w.linear(xq, sx, wq, sw, b, tile=t)) for t in range(w.num_tiles())]
    accs = [w.gemm_i32(xq, wq, tile=t).cpu().numpy() for t in range(w.num_tiles())]
    for t in range(1, len(outs)):
        assert np.array_equal(outs[0], outs[t]) and np.array_equal(accs[0], accs[t]), t


def test_no_writes_outside_outputs(w):
    """Guard bytes around every output buffer stay untouched."""
    M, N, K, G = 77, 136, 320, 4096
    x = datagen.random_bf16((M, K), seed=9).to(DEV)
    W = datagen.random_bf16((N, K), seed=10, std=0.02).to(DEV)
    qbuf = torch.full((M * K + 2 * G,), 0x5A, dtype=torch.int8, device=DEV)
    sbuf = torch.full((M + 2 * G,), 7.0, dtype=torch.float32, device=DEV)
    ybuf = torch.full((M * N + 2 * G,), 0x1234, dtype=torch.int16, device=DEV)
    abuf = torch.full((M * N + 2 * G,), -5, dtype=torch.int32, device=DEV)
    xq = qbuf[G:G + M * K].view(M, K)
    xs = sbuf[G:G + M]
    w.quantize_act(x, xq, xs)
    wq, ws = w.quantize_weight(W)
    y = ybuf[G:G + M * N].view(M, N).view(torch.bfloat16)
    w.linear(xq, xs, wq, ws, None, y=y)
    w.gemm_i32(xq, wq, acc=abuf[G:G + M * N].view(M, N))
    torch.cuda.synchronize()
    for buf, val in ((qbuf, 0x5A), (sbuf, 7.0), (ybuf, 0x1234), (abuf, -5)):
        assert bool((buf[:G] == val).all()) and bool((buf[-G:] == val).all())


def test_empty_m_is_noop(w):
    xq = torch.empty((0, 64), dtype=torch.int8, device=DEV)
    wq = torch.zeros((8, 64), dtype=torch.int8, device=DEV)
    y = w.linear(xq, torch.empty(0, device=DEV), wq, torch.ones(8, device=DEV), None)
    assert y.shape == (0, 8)
    q, s = w.quantize_act(torch.empty((0, 64), dtype=torch.bfloat16, device=DEV))
    assert q.shape == (0, 64) and s.shape == (0,)


def test_errors_raise(w):
    x = torch.zeros((4, 24), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(w.W8A8Error):
        w.quantize_act(x)
    xq = torch.zeros((4, 64), dtype=torch.int8, device=DEV)
    with pytest.raises(w.W8A8Error):
        w.gemm_i32(xq, xq, tile=w.num_tiles())


def test_module_drop_in(w):
    lin = torch.nn.Linear(384, 200, bias=True)
    with torch.no_grad():
        lin.weight.normal_(0, 0.02)
        lin.bias.normal_(0, 0.01)
    lin = lin.to(torch.bfloat16)
    mod = w.W8A8Linear.from_linear(lin.to(DEV))
    x = datagen.random_bf16((3, 17, 384), seed=12)
    y = mod(x.to(DEV))
    assert y.shape == (3, 17, 200) and y.dtype == torch.bfloat16
    ref_wq, ref_ws = quantize_rows_ref(lin.weight.detach().cpu())
    ref_xq, ref_xs = quantize_rows_ref(x.reshape(-1, 384))
    y32 = dequant_ref(int_gemm_ref(ref_xq, ref_wq), ref_xs, ref_ws, lin.bias.detach().cpu())
    assert np.array_equal(bf16_bits(y.reshape(-1, 200)), f32_to_bf16_bits(y32))
