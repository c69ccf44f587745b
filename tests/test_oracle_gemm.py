"""Pins for the oracle's integer GEMM: brute force on tiny shapes, closed
forms, and the int32 overflow bound.  CPU only."""
import numpy as np
import pytest

from datagen import random_int8
from oracle import int_gemm_ref

INT32_MAX = 2 ** 31 - 1
K_BOUND = INT32_MAX // (127 * 127)      # 133144: largest K whose +-127 sums fit int32


def _brute(a, b):
    M, K = a.shape
    N = b.shape[0]
    return [[sum(int(a[m, k]) * int(b[n, k]) for k in range(K)) for n in range(N)] for m in range(M)]


@pytest.mark.parametrize("M,N,K", [(1, 1, 1), (3, 5, 7), (7, 2, 16), (16, 9, 33), (5, 11, 64), (2, 3, 100)])
def test_brute_force_tiny(M, N, K):
    a = random_int8((M, K), seed=M * 100 + N)
    b = random_int8((N, K), seed=K * 7 + 1)
    want = np.array(_brute(a, b), dtype=np.int64)
    assert np.array_equal(int_gemm_ref(a, b, "i64"), want)
    assert np.array_equal(int_gemm_ref(a, b, "i32").astype(np.int64), want)
    # independent library route: numpy int64 matmul against the transpose
    assert np.array_equal(a.astype(np.int64) @ b.astype(np.int64).T, want)


def test_rejects_mismatched_k():
    with pytest.raises(ValueError):
        int_gemm_ref(np.zeros((2, 3), np.int8), np.zeros((2, 4), np.int8))


def test_all_127_closed_form_at_k12288():
    K = 12288
    a = np.full((2, K), 127, np.int8)
    b = np.full((3, K), 127, np.int8)
    b[1] = -127
    c32 = int_gemm_ref(a, b, "i32")
    c64 = int_gemm_ref(a, b, "i64")
    assert np.all(c64[:, 0] == 16129 * K) and 16129 * K == 198193152
    assert np.all(c64[:, 1] == -16129 * K)
    assert np.array_equal(c32.astype(np.int64), c64)


def test_alternating_signs_cancel():
    K = 3072
    a = np.full((1, K), 127, np.int8)
    b = np.tile(np.array([127, -127], np.int8), K // 2)[None, :]
    assert int_gemm_ref(a, b, "i32")[0, 0] == 0


def test_int32_overflow_bound_is_tight():
    """At K = 133144 the extreme sum still fits int32; one more term overflows,
    which the int32 accumulator shows as a wrap-around against int64."""
    assert K_BOUND == 133144
    a = np.full((1, K_BOUND), 127, np.int8)
    assert int_gemm_ref(a, a, "i32")[0, 0] == 16129 * K_BOUND == int_gemm_ref(a, a, "i64")[0, 0]
    a1 = np.full((1, K_BOUND + 1), 127, np.int8)
    exact = 16129 * (K_BOUND + 1)
    assert exact > INT32_MAX
    assert int_gemm_ref(a1, a1, "i64")[0, 0] == exact
    assert int_gemm_ref(a1, a1, "i32")[0, 0] == exact - 2 ** 32
