"""Pins of the fp8 (e4m3) variant's oracle: the e4m3 rounding against a
brute-force nearest search over every code decoded from the format's
definition, exact closed forms of the quantizer, and the accumulation against
exact rational sums."""
from __future__ import annotations

from fractions import Fraction

import numpy as np
import torch

from oracle.fp8 import (e4m3_decode, e4m3_encode, e4m3_round, fp32_sum_bound, fp8_block_sum_bound,
                        fp8_gemm_ref, quantize_rows_fp8_ref, w8a8_fp8_linear_ref)


def _all_codes():
    """(value, code) of every finite non-negative e4m3 number, decoded by hand:
    exponent field 0 -> m/8 * 2^-6, else (1 + m/8) * 2^(e-7); 0x7F is NaN."""
    out = []
    for code in range(0x7F):
        e, m = code >> 3, code & 7
        v = Fraction(m, 8) * Fraction(1, 64) if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
        out.append((v, code))
    return out


def _nearest(x: Fraction, negative: bool):
    """Nearest e4m3 of |x| with ties to the even code; the sign is kept, zero
    included (-0 -> 0x80)."""
    best = None
    for v, c in _all_codes():
        d = abs(abs(x) - v)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, v, c)
    v, c = best[1], best[2]
    if abs(x) >= 464:          # beyond the last rounding boundary: saturate
        v, c = Fraction(448), 0x7E
    return (-v if negative else v), (c | (0x80 if negative else 0))


def test_decode_table():
    vals = [float(v) for v, _ in _all_codes()]
    assert vals[0x7E] == 448.0 and vals[0x01] == 2.0 ** -9 and vals[0x08] == 2.0 ** -6
    codes = np.arange(0x7F, dtype=np.uint8)
    assert np.array_equal(e4m3_decode(codes), np.array(vals))
    assert np.array_equal(e4m3_encode(np.array(vals)), codes)
    assert np.array_equal(e4m3_decode(codes | 0x80), -np.array(vals))


def test_rounding_brute_force():
    rng = np.random.default_rng(8)
    reps = [float(v) for v, _ in _all_codes()]
    mids = [(a + b) / 2 for a, b in zip(reps[:-1], reps[1:])]          # exact ties
    xs = np.concatenate([reps, mids, np.nextafter(mids, 0), np.nextafter(mids, 1e9),
                         rng.uniform(0, 470, 2000), 2.0 ** rng.uniform(-14, 9, 2000),
                         [448.0, 455.9, 456.0, 463.9, 464.0, 1e4]])
    xs = np.concatenate([xs, -xs])
    got_v = e4m3_round(xs)
    got_c = e4m3_encode(got_v)
    for x, gv, gc in zip(xs, got_v, got_c):
        v, c = _nearest(Fraction(float(x)), bool(np.signbit(x)))
        assert gv == float(v) and np.signbit(gv) == np.signbit(x) and int(gc) == c, (x, gv, int(gc), c)


def test_quantizer_closed_form():
    # amax = 448 * 2^e makes s = 2^e exactly; x = v * 2^e for e4m3 values v
    # is then coded exactly, and the amax element gets 0x7E
    vals = np.array([float(v) for v, _ in _all_codes()][:0x7F])
    for e in (-20, 0, 5):
        row = np.concatenate([vals, -vals]) * 2.0 ** e
        x = torch.from_numpy(row.astype(np.float32)[None, :]).to(torch.bfloat16)
        assert np.array_equal(x.float().numpy()[0], row.astype(np.float32))   # exact in bf16
        codes, s = quantize_rows_fp8_ref(x)
        assert s[0] == np.float32(2.0 ** e)
        assert np.array_equal(e4m3_decode(codes[0]), row / 2.0 ** e)
        assert codes[0, 0x7E] == 0x7E


def test_quantizer_zero_row_and_invariants():
    rng = np.random.default_rng(3)
    x = torch.from_numpy(rng.standard_normal((4, 96)).astype(np.float32)).to(torch.bfloat16)
    x[2] = 0
    codes, s = quantize_rows_fp8_ref(x)
    assert s[2] == 0 and not codes[2].any()
    # every non-zero row reaches +-448 at its absmax element
    for r in (0, 1, 3):
        assert np.abs(e4m3_decode(codes[r])).max() == 448.0
    # scaling a row by 2^j leaves the codes unchanged and scales s exactly
    c2, s2 = quantize_rows_fp8_ref(x * 8)
    assert np.array_equal(c2, codes) and np.array_equal(s2, s * 8)


def test_gemm_exact_and_bound():
    rng = np.random.default_rng(4)
    cx = rng.integers(0, 256, size=(3, 40)).astype(np.uint8)
    cw = rng.integers(0, 256, size=(5, 40)).astype(np.uint8)
    cx[cx & 0x7F == 0x7F] = 0   # no NaN codes
    cw[cw & 0x7F == 0x7F] = 0
    acc = fp8_gemm_ref(cx, cw)
    vx, vw = e4m3_decode(cx), e4m3_decode(cw)
    for m in range(3):
        for n in range(5):
            exact = sum(Fraction(float(a)) * Fraction(float(b)) for a, b in zip(vx[m], vw[n]))
            assert Fraction(float(acc[m, n])) == exact
    # a plain left-to-right fp32 sum stays within the bound
    b = fp32_sum_bound(cx, cw)
    for m in range(3):
        for n in range(5):
            s = np.float32(0)
            for a, c in zip(vx[m], vw[n]):
                s = np.float32(s + np.float32(a * c))
            assert abs(float(s) - acc[m, n]) <= b[m, n]


def test_linear_whole_path():
    rng = np.random.default_rng(6)
    x = torch.from_numpy(rng.standard_normal((4, 64)).astype(np.float32)).to(torch.bfloat16)
    w = torch.from_numpy(rng.standard_normal((3, 64)).astype(np.float32) * 0.02).to(torch.bfloat16)
    b = torch.from_numpy(rng.standard_normal(3).astype(np.float32) * 0.01).to(torch.bfloat16)
    r = w8a8_fp8_linear_ref(x, w, b)
    ref = x.double().numpy() @ w.double().numpy().T + b.double().numpy()
    # e4m3 keeps 3 mantissa bits: the product error is a few percent of the scale
    assert np.max(np.abs(r["y32"] - ref)) < 0.1 * np.max(np.abs(ref))


def _aligned_block_gemm(cx, cw, bits: int) -> np.ndarray:
    """Model of a block-summing fp8 unit, computed exactly: per block of 64
    products (exact), every product truncated toward zero below
    2^(E - bits + 1) where 2^E <= max|p| < 2^(E+1), the truncated terms summed
    exactly and rounded to fp32, and the block sums added in fp32 in order."""
    x, w = e4m3_decode(cx), e4m3_decode(cw)
    M, K = x.shape
    N = w.shape[0]
    out = np.zeros((M, N), dtype=np.float32)
    for m in range(M):
        for n in range(N):
            acc = np.float32(0)
            for k0 in range(0, K, 64):
                p = [Fraction(float(a)) * Fraction(float(b)) for a, b in zip(x[m, k0:k0 + 64], w[n, k0:k0 + 64])]
                big = max(abs(v) for v in p)
                if big == 0:
                    continue
                e = 0
                while Fraction(2) ** (e + 1) <= big:
                    e += 1
                while Fraction(2) ** e > big:
                    e -= 1
                q = Fraction(2) ** (e - bits + 1)
                blk = sum((abs(v) // q) * q * (1 if v >= 0 else -1) for v in p)
                acc = np.float32(acc + np.float32(float(blk)))
            out[m, n] = acc
    return out


def test_block_sum_bound_closed_form():
    # K = 64 products of the same magnitude: (2^-15 + 2^-24) * 64 * |p|
    cx = e4m3_encode(np.full((1, 64), 2.0))
    cw = e4m3_encode(np.full((1, 64), -3.0))
    assert fp8_block_sum_bound(cx, cw)[0, 0] == (2.0 ** -15 + 2.0 ** -24) * 64 * 6.0
    # K = 130 -> three blocks of the fp32 term
    cx = e4m3_encode(np.full((2, 130), 0.5))
    cw = e4m3_encode(np.full((1, 130), 1.0))
    assert np.all(fp8_block_sum_bound(cx, cw) == (2.0 ** -15 + 3 * 2.0 ** -24) * 65.0)


def test_block_sum_bound_covers_a_22_bit_block_adder_and_not_a_20_bit_one():
    """The bound holds for the model it states (22 significant bits per
    block), and a 20-bit block adder breaks it on adversarial blocks: one
    large product and 63 small ones whose low bits the alignment drops."""
    rng = np.random.default_rng(5)
    vals = e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    K = 192
    cx = e4m3_encode(rng.choice(np.concatenate([vals, -vals]), (3, K)))
    cw = e4m3_encode(rng.choice(np.concatenate([vals, -vals]), (4, K)))
    # adversarial rows: per block one 448 x 448 product (2^17 <= p < 2^18) and
    # 63 products 0.125 x 1.875 = 0.234375, just under the 20-bit alignment
    # step 2^(17 - 19) = 0.25 (all of it dropped), 3.75 steps of the 22-bit one
    adv_x = np.full(K, 0.125)
    adv_x[::64] = 448.0
    adv_w = np.full(K, 1.875)
    adv_w[::64] = 448.0
    cx = np.vstack([cx, e4m3_encode(adv_x[None, :])])
    cw = np.vstack([cw, e4m3_encode(adv_w[None, :])])
    exact = fp8_gemm_ref(cx, cw)
    bound = fp8_block_sum_bound(cx, cw)
    got22 = _aligned_block_gemm(cx, cw, 22).astype(np.float64)
    assert np.all(np.abs(got22 - exact) <= bound)
    got20 = _aligned_block_gemm(cx, cw, 20).astype(np.float64)
    assert np.any(np.abs(got20 - exact) > bound)
