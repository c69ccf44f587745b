// Row-wise dequantization back to bf16: out[r,k] = bf16_rne(fl32(float(q[r,k]) * scale[r])).
//
// This is the step the abstract of "Realizing Native INT8 Compute for
// Diffusion Transformers on Consumer GPUs" (arXiv 2606.14598) identifies as
// the slow production path: weights and activations are quantized and then
// immediately turned back into bf16 for a bf16 matrix multiply.  It exists
// here so that path can be measured next to the fused int8 GEMM.
//
// HBM-bound: K + 2K bytes per row (+4 for the scale).  Each thread turns 16
// codes (one 16-byte load) into 16 bf16 values (two 16-byte stores), walking
// the matrix with a grid stride; K % 16 == 0 keeps every 16-code chunk
// inside one row.
#include "kernels.h"

namespace w8a8 {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// codes at bytes shift/8 and shift/8 + 1 of word w (sign-extended) -> packed bf16 pair
__device__ __forceinline__ uint32_t pair(uint32_t w, int shift, float s) {
  const float a = (float)(int8_t)(w >> shift);
  const float b = (float)(int8_t)(w >> (shift + 8));
  const bf16x2 v = __builtin_convertvector((f32x2{__fmul_rn(a, s), __fmul_rn(b, s)}), bf16x2);
  return __builtin_bit_cast(uint32_t, v);
}

__global__ __launch_bounds__(256) void dequantize_rows_kernel(const u32x4* __restrict__ q,
                                                              const float* __restrict__ scale,
                                                              u32x4* __restrict__ out,
                                                              int64_t chunks, int64_t chunks_per_row) {
  for (int64_t c = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
       c += (int64_t)gridDim.x * blockDim.x) {
    const float s = scale[c / chunks_per_row];
    const u32x4 v = __builtin_nontemporal_load(q + c);
    u32x4 lo, hi;
    lo[0] = pair(v[0], 0, s);
    lo[1] = pair(v[0], 16, s);
    lo[2] = pair(v[1], 0, s);
    lo[3] = pair(v[1], 16, s);
    hi[0] = pair(v[2], 0, s);
    hi[1] = pair(v[2], 16, s);
    hi[2] = pair(v[3], 0, s);
    hi[3] = pair(v[3], 16, s);
    __builtin_nontemporal_store(lo, out + 2 * c);
    __builtin_nontemporal_store(hi, out + 2 * c + 1);
  }
}

}  // namespace

hipError_t launch_dequantize_rows(const int8_t* q, const float* scale, uint16_t* out, int64_t R,
                                  int64_t K, hipStream_t stream) {
  const int64_t chunks = R * (K / 16);
  constexpr int kThreads = 256;
  // enough workgroups to cover the chunks once, at most 8 resident per CU
  const int64_t want = (chunks + kThreads - 1) / kThreads;
  const unsigned grid = (unsigned)(want < 256 * 8 ? want : 256 * 8);
  hipLaunchKernelGGL(dequantize_rows_kernel, dim3(grid), dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(q), scale, reinterpret_cast<u32x4*>(out),
                     chunks, K / 16);
  return hipGetLastError();
}

}  // namespace w8a8
