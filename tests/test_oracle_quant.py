"""Pins for the oracle's row quantizer (closed forms, exhaustive sweeps,
invariants, and an exact-rational brute force).  CPU only."""
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import bf16_to_f32, quantize_rows_ref
from tests.exact import round_to_f32, rne_int, f32_bits

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _all_finite_bf16_nonneg():
    bits = np.arange(0, 0x7F80, dtype=np.uint16)          # +0 .. largest finite
    return bf16_to_f32(bits)


def test_closed_form_ties_golden():
    rows, expect = [], []
    for line in open(os.path.join(GOLDEN, "quant_closed_form.txt")):
        if line.startswith("#") or not line.strip():
            continue
        lhs, rhs = line.split("|")
        rows.append([float(t) for t in lhs.split()])
        expect.append([int(t) for t in rhs.split()])
    rows = np.array(rows, np.float64)
    expect = np.array(expect, np.int64)
    for e in (-130, -126, -100, -20, -7, 0, 3, 20, 100):
        v = (rows * 2.0 ** e).astype(np.float32)
        assert np.array_equal(v.astype(np.float64), rows * 2.0 ** e)   # exact in fp32 and bf16
        q, s = quantize_rows_ref(v)
        assert np.array_equal(q.astype(np.int64), expect), e
        nz = np.abs(rows).max(axis=1) > 0
        assert np.all(s[nz] == np.float32(2.0 ** e)), e
        assert np.all(s[~nz] == 0)


def test_scale_is_correctly_rounded_exhaustive():
    """s = amax/127 rounded to the nearest fp32, for every finite bf16 amax."""
    amax = _all_finite_bf16_nonneg()[1:]
    v = np.stack([amax, -amax * 0], axis=1).astype(np.float32)
    _, s = quantize_rows_ref(v)
    for a, sv in zip(amax[::7].tolist(), s[::7].tolist()):
        assert sv == round_to_f32(Fraction(a) / 127)
    # vectorised check for all of them: s is the fp32 nearest amax/127
    a64 = amax.astype(np.float64)
    lo = np.nextafter(s, np.float32(0)).astype(np.float64)
    hi = np.nextafter(s, np.float32(np.inf)).astype(np.float64)
    s64 = s.astype(np.float64)
    r = a64 - 127.0 * s64                                      # exact in fp64
    assert np.all(np.abs(r) <= (hi - s64) * 127.0 / 2 + 0)     # within half the upper gap
    assert np.all(-r <= (s64 - lo) * 127.0 / 2)                # and the lower gap


@pytest.mark.parametrize("amax_bits", [0x0001, 0x0080, 0x00FF, 0x3C00, 0x3F80, 0x3F81,
                                       0x3FFF, 0x42FE, 0x4300, 0x4479, 0x5F00, 0x7F7F])
def test_codes_exhaustive_over_all_bf16(amax_bits):
    """For a spread of amax (subnormal to the largest finite), every finite bf16
    x with |x| <= amax: the fp32 quotient is the correctly rounded x/s (checked
    with exact fp64 residuals), the code is its half-even rounding, and codes
    are odd in x."""
    amax = float(bf16_to_f32(np.array([amax_bits], np.uint16))[0])
    allx = _all_finite_bf16_nonneg()
    x = allx[allx <= amax]
    x = np.concatenate([x, -x[1:]]).astype(np.float32)
    row = x.reshape(1, -1)
    q, s = quantize_rows_ref(row)
    q = q[0].astype(np.int64)
    s = s[0]
    assert s == np.float32(amax) / np.float32(127)
    y = (x / s).astype(np.float32)                               # candidate quotient
    # y must be the correctly rounded x/s: x - y*s exact in fp64
    y64, s64, x64 = y.astype(np.float64), np.float64(s), x.astype(np.float64)
    r = x64 - y64 * s64
    up = (np.nextafter(np.abs(y), np.float32(np.inf)).astype(np.float64) - np.abs(y64)) * s64 / 2
    dn = (np.abs(y64) - np.nextafter(np.abs(y), np.float32(0)).astype(np.float64)) * s64 / 2
    ra = np.sign(y64) * r
    nzq = y64 != 0
    assert np.all(np.abs(r[~nzq]) <= up[~nzq])                  # rounds to zero
    assert np.all((ra[nzq] <= up[nzq]) & (-ra[nzq] <= dn[nzq]))  # nearest fp32
    ties = nzq & ((ra == up) | (-ra == dn))
    assert np.all(y.view(np.uint32)[ties] % 2 == 0)               # ties to even
    # half-even rounding of y, written out
    fl = np.floor(y64)
    frac = y64 - fl
    want = np.where(frac > 0.5, fl + 1, np.where(frac < 0.5, fl, np.where(fl % 2 == 0, fl, fl + 1)))
    want = np.clip(want, -127, 127).astype(np.int64)
    assert np.array_equal(q, want)
    # error bound |q*s - x| <= s*(1/2 + 2^-17), oddness, the max hits 127
    assert np.all(np.abs(q * s64 - x64) <= s64 * (0.5 + 2.0 ** -17))
    n = (len(x) + 1) // 2
    assert np.array_equal(q[1:n], -q[n:])
    assert q[np.argmax(np.abs(x))] in (127, -127)


def test_brute_force_exact_rationals():
    """Tiny random rows against exact rational arithmetic."""
    rng = np.random.default_rng(11)
    for trial in range(40):
        K = int(rng.integers(1, 24))
        v32 = (rng.standard_normal((3, K)) * 10.0 ** rng.integers(-6, 6)).astype(np.float32)
        v = torch.from_numpy(v32).to(torch.bfloat16)
        q, s = quantize_rows_ref(v)
        vf = bf16_to_f32(v)
        for r in range(3):
            vals = [Fraction(float(t)) for t in vf[r]]
            amax = max(abs(t) for t in vals)
            sr = round_to_f32(amax / 127)
            assert f32_bits(float(s[r])) == f32_bits(sr)
            for k in range(K):
                quot = round_to_f32(vals[k] / Fraction(sr))
                assert int(q[r, k]) == max(-127, min(127, rne_int(Fraction(quot))))


def test_row_independence_and_permutation():
    """Each row is quantized alone (the reduction runs along K, not M)."""
    rng = np.random.default_rng(5)
    v = (rng.standard_normal((9, 40)) * np.array([1e-3, 1, 50, 1e4, 2, 3, 4, 5, 6])[:, None]).astype(np.float32)
    v = bf16_to_f32(torch.from_numpy(v).to(torch.bfloat16))
    q, s = quantize_rows_ref(v)
    for r in range(9):
        q1, s1 = quantize_rows_ref(v[r:r + 1])
        assert np.array_equal(q1[0], q[r]) and s1[0] == s[r]
    perm = rng.permutation(9)
    qp, sp = quantize_rows_ref(v[perm])
    assert np.array_equal(qp, q[perm]) and np.array_equal(sp, s[perm])
    # the transposed reduction would give different scales here
    assert not np.allclose(s, np.abs(v).max(axis=0)[:9] / 127)


def test_power_of_two_scaling_invariance():
    rng = np.random.default_rng(7)
    v = bf16_to_f32(torch.from_numpy(rng.standard_normal((6, 64)).astype(np.float32)).to(torch.bfloat16))
    q0, s0 = quantize_rows_ref(v)
    for j in (-60, -10, -1, 1, 9, 60):
        q1, s1 = quantize_rows_ref((v * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q0, q1)
        assert np.all(s1 == (s0 * np.float32(2.0 ** j)))


def test_zero_and_negative_max_rows():
    v = np.zeros((3, 16), np.float32)
    v[1, 3] = -5.0
    v[1, 4] = 2.0
    v[2, :] = 1.0
    q, s = quantize_rows_ref(v)
    assert s[0] == 0 and not q[0].any()
    assert q[1, 3] == -127 and s[1] == np.float32(5.0) / np.float32(127)
    assert np.all(q[2] == 127)
    assert not np.isnan(s).any()
