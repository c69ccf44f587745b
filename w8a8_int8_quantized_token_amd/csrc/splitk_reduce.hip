// Second pass of the K-split fused linear: the int32 sums of the K ranges are
// added (exactly -- integer addition, so the result is the accumulator of the
// whole K, acc[m,n] = sum_k xq[m,k] * wq[n,k]) and the per-token x
// per-channel dequantization plus bias of the abstract of "Realizing Native
// INT8 Compute for Diffusion Transformers on Consumer GPUs" (arXiv 2606.14598)
// is applied with the same per-element arithmetic as the fused GEMM's
// epilogue (epilogue.h), so the bf16 output is bit-identical to the fused
// path's.
//
// Bound by memory: each output reads 4 bytes per K range and writes 2.  One
// thread takes 8 consecutive channels of one token: two 16-byte loads per
// range (non-temporal: the slices are read once), one 16-byte store, and the
// channels' scales and bias as 16-byte vectors where they are aligned.
#include "epilogue.h"
#include "kernels.h"

#include <algorithm>

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;

// kVec: channel scales and bias are read as 16-byte vectors (both 16-byte
// aligned); otherwise one element at a time.
template <Epilogue EPI, bool kVec>
__global__ __launch_bounds__(kThreads) void splitk_reduce_kernel(
    const int32_t* __restrict__ part, int chunks, int64_t slice, const float* __restrict__ sx,
    const float* __restrict__ sw, const uint16_t* __restrict__ bias, uint16_t* __restrict__ y,
    int64_t groups_per_row, int64_t groups) {
  for (int64_t g = (int64_t)blockIdx.x * kThreads + threadIdx.x; g < groups;
       g += (int64_t)gridDim.x * kThreads) {
    const int64_t m = g / groups_per_row;
    const int64_t n = (g - m * groups_per_row) * 8;
    const int64_t e0 = m * groups_per_row * 8 + n;   // element index of (m, n) in one slice
    v4i lo = v4i{0, 0, 0, 0}, hi = v4i{0, 0, 0, 0};
    for (int c = 0; c < chunks; ++c) {
      const v4i* p = reinterpret_cast<const v4i*>(part + c * slice + e0);
      lo += __builtin_nontemporal_load(p);
      hi += __builtin_nontemporal_load(p + 1);
    }
    const int acc[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    const float sa = sx[m];
    float swv[8], bv[8];
    if constexpr (kVec) {
      const float4 s0 = *reinterpret_cast<const float4*>(sw + n);
      const float4 s1 = *reinterpret_cast<const float4*>(sw + n + 4);
      swv[0] = s0.x, swv[1] = s0.y, swv[2] = s0.z, swv[3] = s0.w;
      swv[4] = s1.x, swv[5] = s1.y, swv[6] = s1.z, swv[7] = s1.w;
      u32x4 bb = u32x4{0, 0, 0, 0};
      if (bias != nullptr) bb = *reinterpret_cast<const u32x4*>(bias + n);
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        bv[2 * q] = __uint_as_float(bb[q] << 16);
        bv[2 * q + 1] = __uint_as_float(bb[q] & 0xffff0000u);
      }
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        swv[e] = sw[n + e];
        bv[e] = bias != nullptr ? __uint_as_float((uint32_t)bias[n + e] << 16) : 0.0f;
      }
    }
    uint32_t w[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
      float v[2];
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int e = 2 * q + h;
        const float r = dequant((float)acc[e], sa, swv[e], bv[e]);
        v[h] = EPI == Epilogue::kBf16GeluScaleBias ? gelu(r) : r;
      }
      w[q] = __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2{v[0], v[1]}), bf16x2));
    }
    __builtin_nontemporal_store(u32x4{w[0], w[1], w[2], w[3]}, reinterpret_cast<u32x4*>(y + e0));
  }
}

}  // namespace

hipError_t launch_splitk_reduce(Epilogue epi, const int32_t* partials, int chunks, const float* sx,
                                const float* sw, const uint16_t* bias, uint16_t* y, int64_t M,
                                int64_t N, hipStream_t stream) {
  if (N % 8 != 0 || chunks < 1 || epi == Epilogue::kRawI32) return hipErrorInvalidValue;
  const int64_t gpr = N / 8, groups = M * gpr;
  const int64_t blocks = std::min<int64_t>((groups + kThreads - 1) / kThreads, int64_t(1) << 20);
  const bool vec = reinterpret_cast<uintptr_t>(sw) % 16 == 0 &&
                   (bias == nullptr || reinterpret_cast<uintptr_t>(bias) % 16 == 0);
  const dim3 grid((unsigned)blocks), block(kThreads);
  if (epi == Epilogue::kBf16GeluScaleBias) {
    if (vec)
      hipLaunchKernelGGL((splitk_reduce_kernel<Epilogue::kBf16GeluScaleBias, true>), grid, block, 0,
                         stream, partials, chunks, M * N, sx, sw, bias, y, gpr, groups);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<Epilogue::kBf16GeluScaleBias, false>), grid, block, 0,
                         stream, partials, chunks, M * N, sx, sw, bias, y, gpr, groups);
  } else {
    if (vec)
      hipLaunchKernelGGL((splitk_reduce_kernel<Epilogue::kBf16ScaleBias, true>), grid, block, 0, stream,
                         partials, chunks, M * N, sx, sw, bias, y, gpr, groups);
    else
      hipLaunchKernelGGL((splitk_reduce_kernel<Epilogue::kBf16ScaleBias, false>), grid, block, 0,
                         stream, partials, chunks, M * N, sx, sw, bias, y, gpr, groups);
  }
  return hipGetLastError();
}

}  // namespace w8a8
