// C ABI of libw8a8: argument validation, tile selection and launches on the
// caller's stream.  Semantics of each entry point are documented in
// include/w8a8.h.  Validation always completes before anything is launched.
#include "../../include/w8a8.h"
#include "kernels.h"

#include <mutex>

namespace {

constexpr int64_t kMaxRows = int64_t(1) << 26;   // M, N limit (grid size)
constexpr int64_t kMaxQuantK = int64_t(1) << 30;

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) % a) == 0; }

// Shape first; an empty input is then a no-op whatever the pointers are.
w8a8_status check_quant(const uint16_t* x, int64_t R, int64_t K, const int8_t* q, const float* s) {
  if (R < 0 || R > kMaxRows || K < 16 || K % 16 != 0 || K > kMaxQuantK) return W8A8_ERR_SHAPE;
  if (R == 0) return W8A8_OK;
  if (!x || !q || !s) return W8A8_ERR_NULL;
  if (!aligned(x, 16) || !aligned(q, 16) || !aligned(s, 4)) return W8A8_ERR_ALIGN;
  return W8A8_OK;
}

w8a8_status quantize(const uint16_t* x, int64_t R, int64_t K, int8_t* q, float* s,
                     hipStream_t stream) {
  const w8a8_status st = check_quant(x, R, K, q, s);
  if (st != W8A8_OK || R == 0) return st;
  return w8a8::launch_quantize_rows(x, q, s, R, K, stream) == hipSuccess ? W8A8_OK
                                                                          : W8A8_ERR_LAUNCH;
}

w8a8_status check_gemm_shape(int64_t M, int64_t N, int64_t K) {
  if (M < 0 || M > kMaxRows || N < 1 || N > kMaxRows || K < 16 || K % 16 != 0 ||
      K > W8A8_MAX_K)
    return W8A8_ERR_SHAPE;
  return W8A8_OK;
}

w8a8_status check_gemm_ptrs(const int8_t* xq, const int8_t* wq, const void* out) {
  if (!xq || !wq || !out) return W8A8_ERR_NULL;
  if (!aligned(xq, 16) || !aligned(wq, 16)) return W8A8_ERR_ALIGN;
  return W8A8_OK;
}

int resolve_tile(int tile, int64_t M, int64_t N, int64_t K) {
  if (tile < 0) return w8a8::select_tile(M, N, K);
  return tile < w8a8::num_tiles() ? tile : -1;
}

// Scratch of the no-allocation K-split entry point: the int32 slices live in
// this array, which every GPU the library runs on holds (its own copy) until
// the process ends.  In host code `scratch` names a host-side stand-in, not
// the device array: its device address is looked up once per device with
// hipGetSymbolAddress and only that address is ever passed to kernels.
static __device__ __align__(256) int8_t scratch[W8A8_NOALLOC_SCRATCH_BYTES];

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

// Device address of `scratch` on the current device (looked up on the first
// call per device, with that device current).
w8a8_status scratch_ptr(void** out) {
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return W8A8_ERR_LAUNCH;
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return W8A8_ERR_LAUNCH;
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return W8A8_OK;
}

}  // namespace

extern "C" {

const char* w8a8_status_str(w8a8_status s) {
  switch (static_cast<int>(s)) {
    case W8A8_OK: return "ok";
    case W8A8_ERR_NULL: return "a required pointer is NULL";
    case W8A8_ERR_SHAPE: return "shape outside the contract (16 <= K, K % 16 == 0, K <= 133144 for GEMMs, N >= 1, 0 <= M)";
    case W8A8_ERR_ALIGN: return "pointer breaks the alignment contract";
    case W8A8_ERR_LAUNCH: return "HIP kernel launch failed";
    case W8A8_ERR_ARG: return "invalid argument";
    case W8A8_ERR_SCRATCH: return "the request needs more than the no-allocation entry point's 32 MiB scratch";
  }
  return "unknown status";
}

w8a8_status w8a8_quantize_weight(const uint16_t* w, int64_t N, int64_t K, int8_t* wq,
                                 float* w_scale, hipStream_t stream) {
  return quantize(w, N, K, wq, w_scale, stream);
}

w8a8_status w8a8_quantize_act(const uint16_t* x, int64_t M, int64_t K, int8_t* xq,
                              float* x_scale, hipStream_t stream) {
  return quantize(x, M, K, xq, x_scale, stream);
}

w8a8_status w8a8_quantize_weight_fp8(const uint16_t* w, int64_t N, int64_t K, uint8_t* wq,
                                     float* w_scale, hipStream_t stream) {
  const w8a8_status st = check_quant(w, N, K, reinterpret_cast<int8_t*>(wq), w_scale);
  if (st != W8A8_OK || N == 0) return st;
  return w8a8::launch_quantize_rows_fp8(w, wq, w_scale, N, K, stream) == hipSuccess
             ? W8A8_OK
             : W8A8_ERR_LAUNCH;
}

w8a8_status w8a8_quantize_act_fp8(const uint16_t* x, int64_t M, int64_t K, uint8_t* xq,
                                  float* x_scale, hipStream_t stream) {
  return w8a8_quantize_weight_fp8(x, M, K, xq, x_scale, stream);
}

w8a8_status w8a8_dequantize_rows(const int8_t* q, const float* scale, int64_t R, int64_t K,
                                 uint16_t* out, hipStream_t stream) {
  if (R < 0 || R > kMaxRows || K < 16 || K % 16 != 0 || K > kMaxQuantK) return W8A8_ERR_SHAPE;
  if (R == 0) return W8A8_OK;
  if (!q || !scale || !out) return W8A8_ERR_NULL;
  if (!aligned(q, 16) || !aligned(scale, 4) || !aligned(out, 16)) return W8A8_ERR_ALIGN;
  return w8a8::launch_dequantize_rows(q, scale, out, R, K, stream) == hipSuccess ? W8A8_OK
                                                                                 : W8A8_ERR_LAUNCH;
}

}  // extern "C"

namespace {

w8a8_status linear_epi(w8a8::Epilogue epi, const int8_t* xq, const float* x_scale,
                       const int8_t* wq, const float* w_scale, const uint16_t* bias, uint16_t* y,
                       int64_t M, int64_t N, int64_t K, int tile, hipStream_t stream,
                       bool fp8 = false) {
  w8a8_status st = check_gemm_shape(M, N, K);
  if (st != W8A8_OK) return st;
  const int t = resolve_tile(tile, M, N, K);
  if (t < 0) return W8A8_ERR_ARG;
  if (M == 0) return W8A8_OK;
  if (!x_scale || !w_scale) return W8A8_ERR_NULL;
  st = check_gemm_ptrs(xq, wq, y);
  if (st != W8A8_OK) return st;
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(y, 2) ||
      (bias && !aligned(bias, 2)))
    return W8A8_ERR_ALIGN;
  const hipError_t e =
      fp8 ? w8a8::launch_gemm_fp8(t, epi, reinterpret_cast<const uint8_t*>(xq),
                                  reinterpret_cast<const uint8_t*>(wq), x_scale, w_scale, bias, y,
                                  M, N, K, stream)
          : w8a8::launch_gemm(t, epi, xq, wq, x_scale, w_scale, bias, y, M, N, K, stream);
  return e == hipSuccess ? W8A8_OK : W8A8_ERR_LAUNCH;
}

}  // namespace

extern "C" {

w8a8_status w8a8_linear_tile(const int8_t* xq, const float* x_scale, const int8_t* wq,
                             const float* w_scale, const uint16_t* bias, uint16_t* y, int64_t M,
                             int64_t N, int64_t K, int tile, hipStream_t stream) {
  return linear_epi(w8a8::Epilogue::kBf16ScaleBias, xq, x_scale, wq, w_scale, bias, y, M, N, K,
                    tile, stream);
}

w8a8_status w8a8_linear(const int8_t* xq, const float* x_scale, const int8_t* wq,
                        const float* w_scale, const uint16_t* bias, uint16_t* y, int64_t M,
                        int64_t N, int64_t K, hipStream_t stream) {
  return w8a8_linear_tile(xq, x_scale, wq, w_scale, bias, y, M, N, K, -1, stream);
}

w8a8_status w8a8_linear_gelu_tile(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                  const float* w_scale, const uint16_t* bias, uint16_t* y,
                                  int64_t M, int64_t N, int64_t K, int tile, hipStream_t stream) {
  return linear_epi(w8a8::Epilogue::kBf16GeluScaleBias, xq, x_scale, wq, w_scale, bias, y, M, N,
                    K, tile, stream);
}

w8a8_status w8a8_linear_gelu(const int8_t* xq, const float* x_scale, const int8_t* wq,
                             const float* w_scale, const uint16_t* bias, uint16_t* y, int64_t M,
                             int64_t N, int64_t K, hipStream_t stream) {
  return w8a8_linear_gelu_tile(xq, x_scale, wq, w_scale, bias, y, M, N, K, -1, stream);
}

w8a8_status w8a8_gemm_i32_tile(const int8_t* xq, const int8_t* wq, int32_t* acc, int64_t M,
                               int64_t N, int64_t K, int tile, hipStream_t stream) {
  w8a8_status st = check_gemm_shape(M, N, K);
  if (st != W8A8_OK) return st;
  const int t = resolve_tile(tile, M, N, K);
  if (t < 0) return W8A8_ERR_ARG;
  if (M == 0) return W8A8_OK;
  st = check_gemm_ptrs(xq, wq, acc);
  if (st != W8A8_OK) return st;
  if (!aligned(acc, 4)) return W8A8_ERR_ALIGN;
  return w8a8::launch_gemm(t, w8a8::Epilogue::kRawI32, xq, wq, nullptr, nullptr, nullptr, acc, M,
                           N, K, stream) == hipSuccess
             ? W8A8_OK
             : W8A8_ERR_LAUNCH;
}

w8a8_status w8a8_gemm_i32(const int8_t* xq, const int8_t* wq, int32_t* acc, int64_t M, int64_t N,
                          int64_t K, hipStream_t stream) {
  return w8a8_gemm_i32_tile(xq, wq, acc, M, N, K, -1, stream);
}

w8a8_status w8a8_linear_fp8_tile(const uint8_t* xq, const float* x_scale, const uint8_t* wq,
                                 const float* w_scale, const uint16_t* bias, uint16_t* y,
                                 int64_t M, int64_t N, int64_t K, int tile, hipStream_t stream) {
  return linear_epi(w8a8::Epilogue::kBf16ScaleBias, reinterpret_cast<const int8_t*>(xq), x_scale,
                    reinterpret_cast<const int8_t*>(wq), w_scale, bias, y, M, N, K, tile, stream,
                    true);
}

w8a8_status w8a8_linear_fp8(const uint8_t* xq, const float* x_scale, const uint8_t* wq,
                            const float* w_scale, const uint16_t* bias, uint16_t* y, int64_t M,
                            int64_t N, int64_t K, hipStream_t stream) {
  return w8a8_linear_fp8_tile(xq, x_scale, wq, w_scale, bias, y, M, N, K, -1, stream);
}

w8a8_status w8a8_gemm_f32_fp8_tile(const uint8_t* xq, const uint8_t* wq, float* acc, int64_t M,
                                   int64_t N, int64_t K, int tile, hipStream_t stream) {
  w8a8_status st = check_gemm_shape(M, N, K);
  if (st != W8A8_OK) return st;
  const int t = resolve_tile(tile, M, N, K);
  if (t < 0) return W8A8_ERR_ARG;
  if (M == 0) return W8A8_OK;
  st = check_gemm_ptrs(reinterpret_cast<const int8_t*>(xq), reinterpret_cast<const int8_t*>(wq),
                       acc);
  if (st != W8A8_OK) return st;
  if (!aligned(acc, 4)) return W8A8_ERR_ALIGN;
  return w8a8::launch_gemm_fp8(t, w8a8::Epilogue::kRawI32, xq, wq, nullptr, nullptr, nullptr, acc,
                               M, N, K, stream) == hipSuccess
             ? W8A8_OK
             : W8A8_ERR_LAUNCH;
}

w8a8_status w8a8_gemm_f32_fp8(const uint8_t* xq, const uint8_t* wq, float* acc, int64_t M,
                              int64_t N, int64_t K, hipStream_t stream) {
  return w8a8_gemm_f32_fp8_tile(xq, wq, acc, M, N, K, -1, stream);
}

int w8a8_num_tiles(void) { return w8a8::num_tiles(); }

w8a8_status w8a8_tile_info(int tile, int* block_m, int* block_n, int* block_k, int* threads) {
  if (tile < 0 || tile >= w8a8::num_tiles()) return W8A8_ERR_ARG;
  const w8a8::TileDesc& d = w8a8::tile_desc(tile);
  if (block_m) *block_m = d.block_m;
  if (block_n) *block_n = d.block_n;
  if (block_k) *block_k = d.block_k;
  if (threads) *threads = d.threads;
  return W8A8_OK;
}

int w8a8_select_tile(int64_t M, int64_t N, int64_t K) { return w8a8::select_tile(M, N, K); }

int w8a8_select_splitk(int64_t M, int64_t N, int64_t K, int* tile) {
  if (check_gemm_shape(M, N, K) != W8A8_OK) return -1;
  return w8a8::select_splitk(M, N, K, tile);
}

size_t w8a8_linear_splitk_workspace(int64_t M, int64_t N, int splits) {
  if (M < 0 || N < 0 || splits < 1) return 0;
  return splits > 1 ? (size_t)splits * (size_t)M * (size_t)N * sizeof(int32_t) : 0;
}

w8a8_status w8a8_linear_splitk(const int8_t* xq, const float* x_scale, const int8_t* wq,
                               const float* w_scale, const uint16_t* bias, uint16_t* y, int64_t M,
                               int64_t N, int64_t K, int splits, int tile, int gelu,
                               void* workspace, size_t workspace_bytes, hipStream_t stream) {
  w8a8_status st = check_gemm_shape(M, N, K);
  if (st != W8A8_OK) return st;
  if (tile >= w8a8::num_tiles() || splits > 64) return W8A8_ERR_ARG;
  int t = tile;
  if (splits <= 0) {
    int auto_tile = 0;
    splits = w8a8::select_splitk(M, N, K, &auto_tile);
    if (t < 0) t = auto_tile;
  }
  if (t < 0) t = w8a8::select_tile(M, N, K);
  const w8a8::Epilogue epi = gelu ? w8a8::Epilogue::kBf16GeluScaleBias : w8a8::Epilogue::kBf16ScaleBias;
  if (splits == 1) return linear_epi(epi, xq, x_scale, wq, w_scale, bias, y, M, N, K, t, stream);
  if (N % 8 != 0 || K % (16 * splits) != 0) return W8A8_ERR_SHAPE;
  if (M == 0) return W8A8_OK;
  if (!x_scale || !w_scale || !workspace) return W8A8_ERR_NULL;
  st = check_gemm_ptrs(xq, wq, y);
  if (st != W8A8_OK) return st;
  if (!aligned(x_scale, 4) || !aligned(w_scale, 4) || !aligned(y, 16) || !aligned(workspace, 16) ||
      (bias && !aligned(bias, 2)))
    return W8A8_ERR_ALIGN;
  if (workspace_bytes < w8a8_linear_splitk_workspace(M, N, splits)) return W8A8_ERR_ARG;
  int32_t* part = static_cast<int32_t*>(workspace);
  if (w8a8::launch_gemm_partials(t, xq, wq, part, M, N, K, splits, stream) != hipSuccess)
    return W8A8_ERR_LAUNCH;
  return w8a8::launch_splitk_reduce(epi, part, splits, x_scale, w_scale, bias, y, M, N, stream) ==
                 hipSuccess
             ? W8A8_OK
             : W8A8_ERR_LAUNCH;
}

w8a8_status w8a8_linear_splitk_noalloc(const int8_t* xq, const float* x_scale, const int8_t* wq,
                                       const float* w_scale, const uint16_t* bias, uint16_t* y,
                                       int64_t M, int64_t N, int64_t K, int splits, int tile, int gelu,
                                       hipStream_t stream) {
  // the same resolution of `splits` as w8a8_linear_splitk, so the size check
  // below applies to the split that will run
  w8a8_status st = check_gemm_shape(M, N, K);
  if (st != W8A8_OK) return st;
  if (tile >= w8a8::num_tiles() || splits > 64) return W8A8_ERR_ARG;
  if (splits <= 0) {
    int auto_tile = 0;
    splits = w8a8::select_splitk(M, N, K, &auto_tile);
    if (tile < 0) tile = auto_tile;
  }
  const size_t need = w8a8_linear_splitk_workspace(M, N, splits);
  if (need > (size_t)W8A8_NOALLOC_SCRATCH_BYTES) return W8A8_ERR_SCRATCH;
  void* ws = nullptr;
  if (need > 0 && M > 0) {
    st = scratch_ptr(&ws);
    if (st != W8A8_OK) return st;
  }
  return w8a8_linear_splitk(xq, x_scale, wq, w_scale, bias, y, M, N, K, splits, tile, gelu, ws,
                            ws ? (size_t)W8A8_NOALLOC_SCRATCH_BYTES : 0, stream);
}

w8a8_status w8a8_mfma_ceiling(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                              int64_t iters, int64_t* sink, hipStream_t stream) {
  if (M < 256 || M > kMaxRows || N < 192 || N > kMaxRows || K < 128 || K % 16 != 0 ||
      K > W8A8_MAX_K)
    return W8A8_ERR_SHAPE;
  if (iters < 1 || iters > (int64_t(1) << 40)) return W8A8_ERR_ARG;
  if (!xq || !wq || !sink) return W8A8_ERR_NULL;
  if (!aligned(xq, 16) || !aligned(wq, 16) || !aligned(sink, 8)) return W8A8_ERR_ALIGN;
  return w8a8::launch_mfma_ceiling(xq, wq, M, N, K, iters, sink, stream) == hipSuccess
             ? W8A8_OK
             : W8A8_ERR_LAUNCH;
}

}  // extern "C"
