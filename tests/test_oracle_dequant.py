"""Pins for the oracle's epilogue and the whole linear: unit scales, zero rows,
exact power-of-two cases, an error bound against fp64, bf16 rounding, GELU,
and an exact-rational brute force of the whole path on tiny inputs.  CPU only."""
import os
from fractions import Fraction

import numpy as np
import torch

from datagen import random_bf16, random_int8
from oracle import (bf16_to_f32, dequant_ref, dequant_ref64, f32_to_bf16_bits, gelu_ref,
                    int_gemm_ref, quantize_rows_ref, w8a8_linear_ref)
from tests.exact import f32_bits, rne_int, round_to_f32

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def test_unit_scales_zero_bias_return_raw_product():
    a = random_int8((33, 256), seed=1)
    b = random_int8((17, 256), seed=2)
    acc = int_gemm_ref(a, b)
    y = dequant_ref(acc, np.ones(33, np.float32), np.ones(17, np.float32), None)
    assert np.abs(acc).max() < 2 ** 24
    assert np.array_equal(y.astype(np.int64), acc.astype(np.int64))


def test_zero_rows_give_exactly_the_bias():
    x = random_bf16((12, 64), seed=3)
    x[[0, 5, 11]] = 0
    w = random_bf16((20, 64), seed=4, std=0.02)
    b = random_bf16((20,), seed=5, std=0.01)
    r = w8a8_linear_ref(x, w, b)
    bf = bf16_to_f32(b)
    for m in (0, 5, 11):
        assert r["s_a"][m] == 0 and not r["xq"][m].any()
        assert np.array_equal(r["y32"][m], bf)
        assert np.array_equal(r["y_bf16"][m], b.view(torch.int16).numpy().view(np.uint16))
    assert not np.isnan(r["y32"]).any()


def test_power_of_two_scales_exact_and_indexed_right():
    """Distinct power-of-two scales per row and per column make every step
    exact, so the result must equal acc * s_a[m] * s_w[n] + b[n] exactly; a
    swapped index (rows vs columns) or a dropped term breaks it (M != N)."""
    M, N, K = 6, 10, 64
    a = random_int8((M, K), seed=8, lo=-20, hi=20)
    bq = random_int8((N, K), seed=9, lo=-20, hi=20)
    acc = int_gemm_ref(a, bq)
    s_a = np.array([2.0 ** (m % 5 - 2) for m in range(M)], np.float32)
    s_w = np.array([2.0 ** (-(n % 3)) for n in range(N)], np.float32)
    bias = torch.tensor([0.25 * n - 1 for n in range(N)], dtype=torch.bfloat16)
    y = dequant_ref(acc, s_a, s_w, bias)
    for m in range(M):
        for n in range(N):
            exact = Fraction(int(acc[m, n])) * Fraction(float(s_a[m])) * Fraction(float(s_w[n])) \
                + Fraction(0.25 * n - 1)
            assert Fraction(float(y[m, n])) == exact


def test_fp32_epilogue_error_bound_vs_fp64():
    x = random_bf16((64, 512), seed=10)
    w = random_bf16((96, 512), seed=11, std=0.02)
    b = random_bf16((96,), seed=12, std=0.01)
    r = w8a8_linear_ref(x, w, b)
    p = np.abs(r["acc"].astype(np.float64) * r["s_a"].astype(np.float64)[:, None]
               * r["s_w"].astype(np.float64)[None, :])
    bnd = 4.001 * 2.0 ** -24 * (p + np.abs(bf16_to_f32(b)).astype(np.float64)[None, :])
    assert np.all(np.abs(r["y32"].astype(np.float64) - r["y64"]) <= bnd)
    # and the fp64 reference is the same expression
    assert np.array_equal(r["y64"], dequant_ref64(r["acc"], r["s_a"], r["s_w"], b))


def test_bf16_rounding_golden():
    for line in open(os.path.join(GOLDEN, "bf16_rounding.txt")):
        if line.startswith("#") or not line.strip():
            continue
        val, bits = line.split("|")
        got = f32_to_bf16_bits(np.array([float(val)], np.float32))[0]
        assert got == int(bits, 16), (val, hex(got))


def test_gelu_values():
    g = gelu_ref(np.array([0.0, 1.0, -1.0, 8.0, -8.0]))
    assert g[0] == 0.0
    assert abs(g[1] - 0.8413447460685429) < 1e-15           # 1 * Phi(1)
    assert abs(g[2] + 0.15865525393145707) < 1e-15          # -1 * Phi(-1)
    assert abs(g[3] - 8.0) < 1e-12 and abs(g[4]) < 1e-12


def test_gelu_tail_and_symmetry():
    # Phi(-10) = 7.619853024160527e-24 (standard normal tail, 10 sigma)
    g = gelu_ref(np.array([-10.0]))[0]
    assert abs(g / (-10.0 * 7.619853024160527e-24) - 1.0) < 1e-12
    # gelu(v) - gelu(-v) = v * (Phi(v) + Phi(-v)) = v
    v = np.linspace(-6, 6, 97)
    assert np.allclose(gelu_ref(v) - gelu_ref(-v), v, rtol=0, atol=1e-14)


def test_whole_path_brute_force_tiny():
    """Every stage re-derived with exact rationals and explicit fp32 / bf16
    rounding, on tiny inputs."""
    rng = np.random.default_rng(21)
    for trial in range(6):
        M, N, K = int(rng.integers(1, 5)), int(rng.integers(1, 6)), int(rng.integers(1, 20))
        x = random_bf16((M, K), seed=100 + trial)
        w = random_bf16((N, K), seed=200 + trial, std=0.02)
        b = random_bf16((N,), seed=300 + trial, std=0.01)
        r = w8a8_linear_ref(x, w, b)
        xf, wf, bf = bf16_to_f32(x), bf16_to_f32(w), bf16_to_f32(b)

        def quant(row):
            vals = [Fraction(float(t)) for t in row]
            amax = max(abs(t) for t in vals)
            if amax == 0:
                return [0] * len(vals), 0.0
            s = round_to_f32(amax / 127)
            return [max(-127, min(127, rne_int(Fraction(round_to_f32(t / Fraction(s)))))) for t in vals], s

        xq = [quant(xf[m]) for m in range(M)]
        wq = [quant(wf[n]) for n in range(N)]
        for m in range(M):
            assert f32_bits(float(r["s_a"][m])) == f32_bits(xq[m][1])
            for n in range(N):
                acc = sum(xq[m][0][k] * wq[n][0][k] for k in range(K))
                assert int(r["acc"][m, n]) == acc
                t = round_to_f32(Fraction(round_to_f32(Fraction(acc))) * Fraction(xq[m][1]))
                t = round_to_f32(Fraction(t) * Fraction(wq[n][1]))
                y = round_to_f32(Fraction(t) + Fraction(float(bf[n])))
                assert f32_bits(float(r["y32"][m, n])) == f32_bits(y)
