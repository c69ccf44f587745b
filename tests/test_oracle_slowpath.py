"""Pins of the dequantize-to-bf16 oracle (the slow path the fused kernel
replaces, per the abstract of arXiv 2606.14598) against exact arithmetic."""
from __future__ import annotations

import struct
from fractions import Fraction

import numpy as np
import pytest

import oracle
from exact import bf16_value, round_to_bf16, round_to_f32


def _exact_dequant(q: int, s: float) -> float:
    """bf16(fl32(q * s)) from exact rationals and the formats' definitions."""
    return round_to_bf16(Fraction(round_to_f32(Fraction(q) * Fraction(s))))


def _f32(bits: int) -> float:
    return struct.unpack("<f", struct.pack("<I", bits))[0]


def test_exact_rational_random():
    rng = np.random.default_rng(11)
    q = rng.integers(-127, 128, size=(6, 64), dtype=np.int8)
    # scales: typical, large, tiny normal, subnormal fp32 and zero
    s = np.array([0.0173, 3.1e4, 2.0 ** -120 * 1.37, _f32(0x00012345), 0.0, 1.0 + 2.0 ** -8],
                 dtype=np.float32)
    got = oracle.dequant_rows_ref(q, s)
    for r in range(q.shape[0]):
        for k in range(q.shape[1]):
            want = _exact_dequant(int(q[r, k]), float(s[r]))
            assert bf16_value(int(got[r, k])) == want, (r, k, int(q[r, k]), float(s[r]))


def test_power_of_two_scale_is_exact():
    # |q| <= 127 fits the 8-bit bf16 significand, so q * 2^e is representable
    q = np.arange(-127, 128, dtype=np.int8)[None, :]
    for e in (-130, -20, 0, 7, 100):
        got = oracle.dequant_rows_ref(q, np.array([2.0 ** e], dtype=np.float32))
        vals = np.array([bf16_value(int(b)) for b in got[0]])
        assert np.array_equal(vals, q[0].astype(np.float64) * 2.0 ** e)


def test_ties_round_to_even():
    # s = 1 + 2^-8 is exact in fp32; so are the products below (at most 16 bits)
    s = np.array([1.0 + 2.0 ** -8], dtype=np.float32)
    got = oracle.dequant_rows_ref(np.array([[1, 3, -5, 2]], dtype=np.int8), s)
    vals = [bf16_value(int(b)) for b in got[0]]
    # 1.00390625 is halfway between 1 and 1 + 2^-7: ties to the even significand, 1.0
    # 3.01171875 lies between 3.0 and 3.015625 (spacing 2^-6), nearer the latter
    # -5.01953125 lies between -5.0 and -5.03125 (spacing 2^-5), nearer the latter
    # 2.0078125 is halfway between 2.0 and 2.015625: even significand, 2.0
    assert vals == [1.0, 3.015625, -5.03125, 2.0]


def test_zero_scale_gives_signed_zeros():
    got = oracle.dequant_rows_ref(np.array([[5, -5, 0]], dtype=np.int8), np.zeros(1, np.float32))
    assert [int(b) for b in got[0]] == [0x0000, 0x8000, 0x0000]


def test_slow_linear_brute_force():
    rng = np.random.default_rng(5)
    import torch
    M, N, K = 3, 4, 16
    x = torch.from_numpy(rng.standard_normal((M, K)).astype(np.float32)).to(torch.bfloat16)
    wq = rng.integers(-127, 128, size=(N, K), dtype=np.int8)
    s_w = (rng.random(N).astype(np.float32) * np.float32(0.01))
    b = torch.from_numpy(rng.standard_normal(N).astype(np.float32) * np.float32(0.1)).to(torch.bfloat16)
    r = oracle.dequant_bf16_linear_ref(x, wq, s_w, b)
    xq, s_a = oracle.quantize_rows_ref(x)
    bf = b.view(torch.int16).numpy().view(np.uint16)
    for m in range(M):
        for n in range(N):
            acc = Fraction(0)
            for k in range(K):
                acc += Fraction(_exact_dequant(int(xq[m, k]), float(s_a[m]))) * \
                    Fraction(_exact_dequant(int(wq[n, k]), float(s_w[n])))
            acc += Fraction(bf16_value(int(bf[n])))
            assert r["y64"][m, n] == pytest.approx(float(acc), rel=1e-14, abs=1e-300)
