// Host-side checks of the libw8a8 C ABI for a build with the address and
// undefined-behaviour sanitizers on the host code: every argument-validation
// path of include/w8a8.h returns its documented status before anything is
// launched, and the per-shape plan choice runs over a grid of shapes.  No
// GPU is touched: no call below reaches a launch (the pointers are never
// dereferenced).  Exit status 0 when every check passes.
#include <cstdint>
#include <cstdio>
#include <cstring>

#include "../../include/w8a8.h"

namespace {

int failures = 0;

void expect(int got, int want, const char* what, int line) {
  if (got != want) {
    std::fprintf(stderr, "line %d: %s returned %d, expected %d\n", line, what, got, want);
    ++failures;
  }
}
#define EXPECT(call, want) expect((int)(call), (want), #call, __LINE__)

// fake device addresses, 16-byte aligned, never dereferenced
void* const A = reinterpret_cast<void*>(uintptr_t(0x10000));
template <class T>
T* p(uintptr_t off = 0) {
  return reinterpret_cast<T*>(reinterpret_cast<uintptr_t>(A) + off);
}

typedef w8a8_status (*QuantFn)(const uint16_t*, int64_t, int64_t, int8_t*, float*, hipStream_t);
typedef w8a8_status (*QuantFp8Fn)(const uint16_t*, int64_t, int64_t, uint8_t*, float*, hipStream_t);

template <class Q, class F>
void check_quantizer(F f) {
  EXPECT(f(nullptr, 4, 64, p<Q>(), p<float>(), nullptr), W8A8_ERR_NULL);
  EXPECT(f(p<uint16_t>(), 4, 64, nullptr, p<float>(), nullptr), W8A8_ERR_NULL);
  EXPECT(f(p<uint16_t>(), 4, 64, p<Q>(), nullptr, nullptr), W8A8_ERR_NULL);
  const int64_t bad[][2] = {{-1, 64}, {4, 0}, {4, 8}, {4, 24}, {4, 15}, {INT64_MIN, 64}, {4, INT64_MAX}};
  for (const auto& rk : bad) EXPECT(f(p<uint16_t>(), rk[0], rk[1], p<Q>(), p<float>(), nullptr), W8A8_ERR_SHAPE);
  EXPECT(f(p<uint16_t>(2), 4, 64, p<Q>(), p<float>(), nullptr), W8A8_ERR_ALIGN);
  EXPECT(f(p<uint16_t>(), 4, 64, p<Q>(8), p<float>(), nullptr), W8A8_ERR_ALIGN);
  EXPECT(f(p<uint16_t>(), 4, 64, p<Q>(), p<float>(2), nullptr), W8A8_ERR_ALIGN);
  EXPECT(f(p<uint16_t>(), 0, 64, p<Q>(), p<float>(), nullptr), W8A8_OK);
  EXPECT(f(nullptr, 0, 64, nullptr, nullptr, nullptr), W8A8_OK);
}

template <class C, class L>
void check_linear(L f) {
  const C* x = p<C>();
  const C* w = p<C>();
  const float* s = p<float>();
  const uint16_t* b = p<uint16_t>();
  uint16_t* y = p<uint16_t>();
  EXPECT(f(nullptr, s, w, s, b, y, 8, 8, 64, nullptr), W8A8_ERR_NULL);
  EXPECT(f(x, s, nullptr, s, b, y, 8, 8, 64, nullptr), W8A8_ERR_NULL);
  EXPECT(f(x, s, w, s, b, nullptr, 8, 8, 64, nullptr), W8A8_ERR_NULL);
  EXPECT(f(x, nullptr, w, s, b, y, 8, 8, 64, nullptr), W8A8_ERR_NULL);
  EXPECT(f(x, s, w, nullptr, b, y, 8, 8, 64, nullptr), W8A8_ERR_NULL);
  const int64_t bad[][3] = {{-1, 8, 64}, {8, 0, 64}, {8, 8, 0}, {8, 8, 8}, {8, 8, 40}, {8, 8, 133152},
                            {INT64_MAX, 8, 64}, {8, INT64_MAX, 64}, {8, 8, INT64_MIN}};
  for (const auto& s3 : bad) EXPECT(f(x, s, w, s, b, y, s3[0], s3[1], s3[2], nullptr), W8A8_ERR_SHAPE);
  EXPECT(f(p<C>(4), s, w, s, b, y, 8, 8, 64, nullptr), W8A8_ERR_ALIGN);
  EXPECT(f(x, s, p<C>(1), s, b, y, 8, 8, 64, nullptr), W8A8_ERR_ALIGN);
  EXPECT(f(x, s, w, s, b, p<uint16_t>(1), 8, 8, 64, nullptr), W8A8_ERR_ALIGN);
  EXPECT(f(x, s, w, s, p<uint16_t>(1), y, 8, 8, 64, nullptr), W8A8_ERR_ALIGN);
  EXPECT(f(x, p<float>(2), w, s, b, y, 8, 8, 64, nullptr), W8A8_ERR_ALIGN);
  EXPECT(f(x, s, w, s, b, y, 0, 8, 64, nullptr), W8A8_OK);
  EXPECT(f(x, s, w, s, nullptr, y, 0, 8, 64, nullptr), W8A8_OK);
  EXPECT(f(nullptr, nullptr, w, s, b, nullptr, 0, 8, 64, nullptr), W8A8_OK);
}

}  // namespace

int main() {
  // status strings
  for (int st = 0; st < 6; ++st)
    if (std::strlen(w8a8_status_str((w8a8_status)st)) == 0) ++failures;
  if (std::strcmp(w8a8_status_str(W8A8_OK), "ok") != 0) ++failures;
  if (!std::strstr(w8a8_status_str((w8a8_status)77), "unknown")) ++failures;

  check_quantizer<int8_t>(static_cast<QuantFn>(w8a8_quantize_weight));
  check_quantizer<int8_t>(static_cast<QuantFn>(w8a8_quantize_act));
  check_quantizer<uint8_t>(static_cast<QuantFp8Fn>(w8a8_quantize_weight_fp8));
  check_quantizer<uint8_t>(static_cast<QuantFp8Fn>(w8a8_quantize_act_fp8));
  check_linear<int8_t>(w8a8_linear);
  check_linear<int8_t>(w8a8_linear_gelu);
  check_linear<uint8_t>(w8a8_linear_fp8);

  const int nt = w8a8_num_tiles();
  EXPECT(nt >= 2, 1);
  const int8_t* q = p<int8_t>();
  const float* s = p<float>();
  EXPECT(w8a8_linear_tile(q, s, q, s, p<uint16_t>(), p<uint16_t>(), 0, 8, 64, 99, nullptr), W8A8_ERR_ARG);
  EXPECT(w8a8_linear_tile(q, s, q, s, p<uint16_t>(), p<uint16_t>(), 0, 8, 64, nt, nullptr), W8A8_ERR_ARG);
  EXPECT(w8a8_linear_gelu_tile(q, s, q, s, nullptr, p<uint16_t>(), 0, 8, 64, nt, nullptr), W8A8_ERR_ARG);

  // raw accumulator entries
  EXPECT(w8a8_gemm_i32(nullptr, q, p<int32_t>(), 8, 8, 64, nullptr), W8A8_ERR_NULL);
  EXPECT(w8a8_gemm_i32(q, q, nullptr, 8, 8, 64, nullptr), W8A8_ERR_NULL);
  EXPECT(w8a8_gemm_i32(q, q, p<int32_t>(), 8, 8, W8A8_MAX_K + 16, nullptr), W8A8_ERR_SHAPE);
  EXPECT(w8a8_gemm_i32(q, q, p<int32_t>(2), 8, 8, 64, nullptr), W8A8_ERR_ALIGN);
  EXPECT(w8a8_gemm_i32(q, q, p<int32_t>(), 0, 8, 133136, nullptr), W8A8_OK);
  EXPECT(w8a8_gemm_i32_tile(q, q, p<int32_t>(), 0, 8, 64, -7, nullptr), W8A8_OK);
  EXPECT(w8a8_gemm_i32_tile(q, q, p<int32_t>(), 0, 8, 64, 99, nullptr), W8A8_ERR_ARG);
  const uint8_t* f8 = p<uint8_t>();
  EXPECT(w8a8_gemm_f32_fp8(nullptr, f8, p<float>(), 8, 8, 64, nullptr), W8A8_ERR_NULL);
  EXPECT(w8a8_gemm_f32_fp8(f8, f8, p<float>(2), 8, 8, 64, nullptr), W8A8_ERR_ALIGN);
  EXPECT(w8a8_gemm_f32_fp8_tile(f8, f8, p<float>(), 0, 8, 64, 99, nullptr), W8A8_ERR_ARG);
  EXPECT(w8a8_linear_fp8_tile(f8, s, f8, s, nullptr, p<uint16_t>(), 0, 8, 64, 99, nullptr), W8A8_ERR_ARG);

  // dequantization
  EXPECT(w8a8_dequantize_rows(nullptr, s, 4, 64, p<uint16_t>(), nullptr), W8A8_ERR_NULL);
  EXPECT(w8a8_dequantize_rows(q, s, 4, 24, p<uint16_t>(), nullptr), W8A8_ERR_SHAPE);
  EXPECT(w8a8_dequantize_rows(p<int8_t>(8), s, 4, 64, p<uint16_t>(), nullptr), W8A8_ERR_ALIGN);
  EXPECT(w8a8_dequantize_rows(nullptr, nullptr, 0, 64, nullptr, nullptr), W8A8_OK);

  // tile table and plan choice over a grid of shapes (host arithmetic only)
  for (int t = 0; t < nt; ++t) {
    int bm = 0, bn = 0, bk = 0, th = 0;
    EXPECT(w8a8_tile_info(t, &bm, &bn, &bk, &th), W8A8_OK);
    if (bm % 32 || bn % 32 || bk % 32 || th % 64) ++failures;
    EXPECT(w8a8_tile_info(t, nullptr, nullptr, nullptr, nullptr), W8A8_OK);
  }
  EXPECT(w8a8_tile_info(nt, nullptr, nullptr, nullptr, nullptr), W8A8_ERR_ARG);
  EXPECT(w8a8_tile_info(-1, nullptr, nullptr, nullptr, nullptr), W8A8_ERR_ARG);
  const int64_t ms[] = {1, 2, 63, 64, 255, 256, 2304, 4096, 8191, 8192, 65536, int64_t(1) << 26};
  const int64_t ns[] = {1, 16, 127, 3072, 9216, 12288, 50000, int64_t(1) << 26};
  const int64_t ks[] = {16, 256, 3072, 12288, W8A8_MAX_K - 8};
  for (int64_t m : ms)
    for (int64_t n : ns)
      for (int64_t k : ks) {
        const int t = w8a8_select_tile(m, n, k);
        if (t < 0 || t >= nt) {
          std::fprintf(stderr, "select_tile(%lld, %lld, %lld) = %d\n", (long long)m, (long long)n,
                       (long long)k, t);
          ++failures;
        }
      }

  // matrix-core ceiling diagnostic: validation only
  int64_t* sk = p<int64_t>();
  EXPECT(w8a8_mfma_ceiling(q, q, 255, 192, 128, 1, sk, nullptr), W8A8_ERR_SHAPE);
  EXPECT(w8a8_mfma_ceiling(q, q, 256, 191, 128, 1, sk, nullptr), W8A8_ERR_SHAPE);
  EXPECT(w8a8_mfma_ceiling(q, q, 256, 192, 112, 1, sk, nullptr), W8A8_ERR_SHAPE);
  EXPECT(w8a8_mfma_ceiling(q, q, 256, 192, 136, 1, sk, nullptr), W8A8_ERR_SHAPE);
  EXPECT(w8a8_mfma_ceiling(q, q, 256, 192, 128, 0, sk, nullptr), W8A8_ERR_ARG);
  EXPECT(w8a8_mfma_ceiling(q, q, 256, 192, 128, (int64_t(1) << 40) + 1, sk, nullptr), W8A8_ERR_ARG);
  EXPECT(w8a8_mfma_ceiling(nullptr, q, 256, 192, 128, 1, sk, nullptr), W8A8_ERR_NULL);
  EXPECT(w8a8_mfma_ceiling(q, q, 256, 192, 128, 1, nullptr, nullptr), W8A8_ERR_NULL);
  EXPECT(w8a8_mfma_ceiling(p<int8_t>(8), q, 256, 192, 128, 1, sk, nullptr), W8A8_ERR_ALIGN);
  EXPECT(w8a8_mfma_ceiling(q, q, 256, 192, 128, 1, p<int64_t>(4), nullptr), W8A8_ERR_ALIGN);

  if (failures) {
    std::fprintf(stderr, "%d check(s) failed\n", failures);
    return 1;
  }
  std::printf("abi host checks ok (%d tile plans)\n", nt);
  return 0;
}
