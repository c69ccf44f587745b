/* Plain integer GEMM for the oracle (test infrastructure only).
 *
 * c[m][n] = sum_k a[m][k] * b[n][k], with a = int8 activations [M,K] and
 * b = int8 weights [N,K], both K-contiguous, as in the int8 x int8 -> int32
 * accumulation described in the abstract of "Realizing Native INT8 Compute for
 * Diffusion Transformers on Consumer GPUs" (arXiv 2606.14598).
 *
 * The int32 variant accumulates modulo 2^32 in uint32_t (well-defined wrap
 * around) and converts back to int32, so an overflow shows up as a mismatch
 * against the int64 variant instead of undefined behaviour.  Integer sums are
 * exact, so the loop order is irrelevant; rows are split across OpenMP threads.
 */
#include <stdint.h>

void oracle_int_gemm_i32(const int8_t *a, const int8_t *b, int32_t *c,
                         int64_t M, int64_t N, int64_t K) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++) {
    const int8_t *ar = a + m * K;
    for (int64_t n = 0; n < N; n++) {
      const int8_t *br = b + n * K;
      uint32_t acc = 0;
      for (int64_t k = 0; k < K; k++)
        acc += (uint32_t)((int32_t)ar[k] * (int32_t)br[k]);
      c[m * N + n] = (int32_t)acc;
    }
  }
}

void oracle_int_gemm_i64(const int8_t *a, const int8_t *b, int64_t *c,
                         int64_t M, int64_t N, int64_t K) {
#pragma omp parallel for schedule(static)
  for (int64_t m = 0; m < M; m++) {
    const int8_t *ar = a + m * K;
    for (int64_t n = 0; n < N; n++) {
      const int8_t *br = b + n * K;
      int64_t acc = 0;
      for (int64_t k = 0; k < K; k++)
        acc += (int64_t)ar[k] * (int64_t)br[k];
      c[m * N + n] = acc;
    }
  }
}
