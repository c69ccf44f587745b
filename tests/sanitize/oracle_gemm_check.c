/* Checks of the oracle's plain C integer GEMM (oracle/int_gemm.c) for a
 * build with the address and undefined-behaviour sanitizers: both
 * accumulation modes against a direct triple loop on small ragged shapes,
 * the all-127 closed form 16129*K at K = 12288, the largest K whose sums fit
 * int32 (133144: exact in both modes), the first K that wraps (133145: the
 * int32 mode returns 16129*K - 2^32), and alternating signs cancelling to 0.
 * Exit status 0 when every check passes. */
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>

void oracle_int_gemm_i32(const int8_t *a, const int8_t *b, int32_t *c, int64_t M, int64_t N, int64_t K);
void oracle_int_gemm_i64(const int8_t *a, const int8_t *b, int64_t *c, int64_t M, int64_t N, int64_t K);

static int failures = 0;
static uint64_t state = 0x9e3779b97f4a7c15ull;

static int8_t rand_code(void) {
  state = state * 6364136223846793005ull + 1442695040888963407ull;
  return (int8_t)((int)((state >> 33) % 255u) - 127);
}

static void small_shapes(void) {
  const int64_t shapes[][3] = {{1, 1, 16}, {3, 5, 32}, {7, 2, 48}, {17, 9, 80}, {33, 31, 256}};
  for (size_t s = 0; s < sizeof shapes / sizeof shapes[0]; ++s) {
    const int64_t M = shapes[s][0], N = shapes[s][1], K = shapes[s][2];
    int8_t *a = malloc((size_t)(M * K)), *b = malloc((size_t)(N * K));
    int32_t *c32 = malloc(sizeof(int32_t) * (size_t)(M * N));
    int64_t *c64 = malloc(sizeof(int64_t) * (size_t)(M * N));
    for (int64_t i = 0; i < M * K; ++i) a[i] = rand_code();
    for (int64_t i = 0; i < N * K; ++i) b[i] = rand_code();
    oracle_int_gemm_i32(a, b, c32, M, N, K);
    oracle_int_gemm_i64(a, b, c64, M, N, K);
    for (int64_t m = 0; m < M; ++m)
      for (int64_t n = 0; n < N; ++n) {
        int64_t want = 0;
        for (int64_t k = 0; k < K; ++k) want += (int64_t)a[m * K + k] * b[n * K + k];
        if (c64[m * N + n] != want || c32[m * N + n] != (int32_t)want) {
          fprintf(stderr, "shape %lldx%lldx%lld (%lld,%lld): %lld / %d, want %lld\n", (long long)M,
                  (long long)N, (long long)K, (long long)m, (long long)n, (long long)c64[m * N + n],
                  c32[m * N + n], (long long)want);
          ++failures;
        }
      }
    free(a); free(b); free(c32); free(c64);
  }
}

/* one row of all 127 (or alternating +-127) times two such channels */
static void closed_form(int64_t K, int alternate, int64_t want64, int32_t want32) {
  int8_t *a = malloc((size_t)K), *b = malloc((size_t)(2 * K));
  for (int64_t k = 0; k < K; ++k) {
    a[k] = 127;
    b[k] = b[K + k] = (int8_t)(alternate && (k & 1) ? -127 : 127);
  }
  int32_t c32[2];
  int64_t c64[2];
  oracle_int_gemm_i32(a, b, c32, 1, 2, K);
  oracle_int_gemm_i64(a, b, c64, 1, 2, K);
  for (int n = 0; n < 2; ++n)
    if (c64[n] != want64 || c32[n] != want32) {
      fprintf(stderr, "K=%lld alternate=%d: %lld / %d, want %lld / %d\n", (long long)K, alternate,
              (long long)c64[n], c32[n], (long long)want64, want32);
      ++failures;
    }
  free(a); free(b);
}

int main(void) {
  small_shapes();
  closed_form(12288, 0, 16129ll * 12288, (int32_t)(16129ll * 12288));
  closed_form(133144, 0, 16129ll * 133144, (int32_t)(16129ll * 133144));
  closed_form(133145, 0, 16129ll * 133145, (int32_t)(16129ll * 133145 - 4294967296ll));
  closed_form(12288, 1, 0, 0);
  if (failures) {
    fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  printf("oracle gemm checks ok\n");
  return 0;
}
