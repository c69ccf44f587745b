// Per-row absmax int8 quantizer for gfx950: per-token activation quantization
// and per-output-channel weight quantization, as in the abstract of
// "Realizing Native INT8 Compute for Diffusion Transformers on Consumer GPUs"
// (arXiv 2606.14598), with the readings s = fl32(amax/127) and
// q = clamp(rne(fl32(x/s)), -127, 127); an all-zero row gives s = 0, q = 0.
//
// One wavefront owns one row.  The row is read once from HBM with 16-byte
// loads (8 bf16 per lane per load) and kept in registers; the absmax is a
// packed 16-bit integer max over the magnitude bits (for finite bf16 the
// order of |x| equals the order of its bits) followed by a wavefront
// butterfly; the codes are then produced from the registers and written with
// 8-byte stores.  HBM traffic is the algorithmic 3 bytes per element plus
// 4 bytes per row.
//
// Division: the codes need rne(fl32(x/s)) exactly.  Instead of a full IEEE
// division per element the kernel computes r = fl32(1/s) once per row and
//   q0 = fl32(x*r), e = fma(-q0, s, x), q = fma(e, r, q0)
// (one Markstein correction step).  Rows with s < 2^-100 first scale x and s
// by 2^100, which is exact and keeps 1/s finite.  An exhaustive host check
// over every finite bf16 (x, amax) pair with |x| <= amax shows the resulting
// codes equal those of the correctly rounded quotient.
//
// The fp8 variant (F8) is the same kernel with s = fl32(amax/448) and codes
// e4m3(fl32(x/s)) (OCP e4m3: nearest, ties to even, largest value 448)
// produced by v_cvt_pk_fp8_f32; the same exhaustive check covers its codes.
#include "kernels.h"

namespace w8a8 {
namespace {

constexpr int kWave = 64;
constexpr int kRowsPerBlock = 4;
constexpr int kThreads = kWave * kRowsPerBlock;

typedef unsigned short ushort2_t __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

__device__ __forceinline__ uint32_t wave_max(uint32_t v) {
#pragma unroll
  for (int off = 32; off > 0; off >>= 1) v = max(v, (uint32_t)__shfl_xor((int)v, off, kWave));
  return v;
}

__device__ __forceinline__ uint32_t absmax_bits(uint32_t acc, uint32_t w) {
  // packed max of the two 15-bit magnitudes held in one 32-bit word
  ushort2_t a = __builtin_bit_cast(ushort2_t, acc);
  ushort2_t b = __builtin_bit_cast(ushort2_t, w & 0x7fff7fffu);
  return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(a, b));
}

__device__ __forceinline__ int code(float x, float s, float r) {
  float q0 = x * r;
  float e = __builtin_fmaf(-q0, s, x);
  float q = __builtin_fmaf(e, r, q0);
  q = __builtin_rintf(q);
  q = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
  return (int)q;
}

// fp8 variant: the quotient fl32(x/s) itself, for the e4m3 conversion; the
// clamp only guards the last fp32 rounding of |x/s| <= 448.  The correction
// step turns x = -0 into +0 (-0 + +0 = +0), and e4m3 keeps the sign of zero,
// so the sign is copied back from x (s > 0: x/s has the sign of x).
__device__ __forceinline__ float quot(float x, float s, float r) {
  const float q0 = x * r;
  const float e = __builtin_fmaf(-q0, s, x);
  const float q = __builtin_fminf(__builtin_fmaxf(__builtin_fmaf(e, r, q0), -448.0f), 448.0f);
  return __builtin_copysignf(q, x);
}

__device__ __forceinline__ uint32_t pack4(int a, int b, int c, int d) {
  return (uint32_t)(a & 0xff) | ((uint32_t)(b & 0xff) << 8) | ((uint32_t)(c & 0xff) << 16) |
         ((uint32_t)d << 24);
}

// 8 bf16 (one 16-byte chunk) -> 8 codes (8 bytes); xs scales x (1 or 2^100).
template <bool F8>
__device__ __forceinline__ u32x2 quant_chunk(u32x4 v, float xs, float s, float r) {
  uint32_t w[4] = {v.x, v.y, v.z, v.w};
  if constexpr (F8) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      f[2 * i] = quot(__uint_as_float(w[i] << 16) * xs, s, r);
      f[2 * i + 1] = quot(__uint_as_float(w[i] & 0xffff0000u) * xs, s, r);
    }
    int lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[0], f[1], 0, false);
    lo = __builtin_amdgcn_cvt_pk_fp8_f32(f[2], f[3], lo, true);
    int hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[4], f[5], 0, false);
    hi = __builtin_amdgcn_cvt_pk_fp8_f32(f[6], f[7], hi, true);
    return u32x2{(uint32_t)lo, (uint32_t)hi};
  }
  int c[8];
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    c[2 * i] = code(__uint_as_float(w[i] << 16) * xs, s, r);
    c[2 * i + 1] = code(__uint_as_float(w[i] & 0xffff0000u) * xs, s, r);
  }
  return u32x2{pack4(c[0], c[1], c[2], c[3]), pack4(c[4], c[5], c[6], c[7])};
}

struct RowScale {
  float s;   // stored scale fl32(amax/127) (fp8: /448), 0 for a zero row
  float ss;  // scale used in the division (s, or s*2^100)
  float xs;  // factor applied to x (1 or 2^100)
  float r;   // fl32(1/ss)
};

template <bool F8>
__device__ __forceinline__ RowScale row_scale(uint32_t amax_bits) {
  RowScale rs;
  float amax = __uint_as_float(amax_bits << 16);
  rs.s = amax / (F8 ? 448.0f : 127.0f);  // correctly rounded (IEEE division)
  rs.xs = 1.0f;
  rs.ss = rs.s;
  if (rs.s < 0x1p-100f) {
    rs.xs = 0x1p100f;
    rs.ss = rs.s * 0x1p100f;
  }
  rs.r = 1.0f / rs.ss;   // correctly rounded
  return rs;
}

// Row resident in registers: CPL 16-byte chunks per lane, K <= CPL*8*64.
template <int CPL, bool F8>
__global__ __launch_bounds__(kThreads) void quantize_rows_reg(const u32x4* __restrict__ x,
                                                              u32x2* __restrict__ q,
                                                              float* __restrict__ scale,
                                                              int64_t R, int nchunk) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= R) return;  // whole wavefront leaves together
  const u32x4* xr = x + row * nchunk;
  u32x2* qr = q + row * nchunk;

  u32x4 v[CPL];
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + i * kWave;
    v[i] = c < nchunk ? __builtin_nontemporal_load(xr + c) : u32x4{0, 0, 0, 0};
  }
  uint32_t m = 0;
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    m = absmax_bits(m, v[i].x);
    m = absmax_bits(m, v[i].y);
    m = absmax_bits(m, v[i].z);
    m = absmax_bits(m, v[i].w);
  }
  m = max(m & 0xffffu, m >> 16);
  m = wave_max(m);

  if (m == 0) {
#pragma unroll
    for (int i = 0; i < CPL; ++i) {
      const int c = lane + i * kWave;
      if (c < nchunk) qr[c] = u32x2{0, 0};
    }
    if (lane == 0) scale[row] = 0.0f;
    return;
  }
  const RowScale rs = row_scale<F8>(m);
#pragma unroll
  for (int i = 0; i < CPL; ++i) {
    const int c = lane + i * kWave;
    if (c < nchunk) qr[c] = quant_chunk<F8>(v[i], rs.xs, rs.ss, rs.r);
  }
  if (lane == 0) scale[row] = rs.s;
}

// Any K: two passes over the row (the second one mostly from cache).
template <bool F8>
__global__ __launch_bounds__(kThreads) void quantize_rows_2pass(const u32x4* __restrict__ x,
                                                                u32x2* __restrict__ q,
                                                                float* __restrict__ scale,
                                                                int64_t R, int nchunk) {
  const int lane = threadIdx.x % kWave;
  const int64_t row = (int64_t)blockIdx.x * kRowsPerBlock + threadIdx.x / kWave;
  if (row >= R) return;
  const u32x4* xr = x + row * nchunk;
  u32x2* qr = q + row * nchunk;
  uint32_t m = 0;
  for (int c = lane; c < nchunk; c += kWave) {
    u32x4 v = xr[c];
    m = absmax_bits(m, v.x);
    m = absmax_bits(m, v.y);
    m = absmax_bits(m, v.z);
    m = absmax_bits(m, v.w);
  }
  m = max(m & 0xffffu, m >> 16);
  m = wave_max(m);
  if (m == 0) {
    for (int c = lane; c < nchunk; c += kWave) qr[c] = u32x2{0, 0};
    if (lane == 0) scale[row] = 0.0f;
    return;
  }
  const RowScale rs = row_scale<F8>(m);
  for (int c = lane; c < nchunk; c += kWave) qr[c] = quant_chunk<F8>(xr[c], rs.xs, rs.ss, rs.r);
  if (lane == 0) scale[row] = rs.s;
}

template <int CPL, bool F8>
hipError_t launch_reg(const uint16_t* x, int8_t* q, float* s, int64_t R, int nchunk,
                      hipStream_t st) {
  const int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((quantize_rows_reg<CPL, F8>), dim3((unsigned)blocks), dim3(kThreads), 0, st,
                     reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x2*>(q), s, R, nchunk);
  return hipGetLastError();
}

template <bool F8>
hipError_t launch_rows(const uint16_t* x, int8_t* q, float* scale, int64_t R, int64_t K,
                       hipStream_t stream) {
  const int nchunk = (int)(K / 8);          // 16-byte chunks per row
  const int cpl = (nchunk + kWave - 1) / kWave;
  if (cpl <= 1) return launch_reg<1, F8>(x, q, scale, R, nchunk, stream);
  if (cpl <= 2) return launch_reg<2, F8>(x, q, scale, R, nchunk, stream);
  if (cpl <= 4) return launch_reg<4, F8>(x, q, scale, R, nchunk, stream);
  if (cpl <= 6) return launch_reg<6, F8>(x, q, scale, R, nchunk, stream);
  if (cpl <= 8) return launch_reg<8, F8>(x, q, scale, R, nchunk, stream);
  if (cpl <= 12) return launch_reg<12, F8>(x, q, scale, R, nchunk, stream);
  if (cpl <= 16) return launch_reg<16, F8>(x, q, scale, R, nchunk, stream);
  if (cpl <= 24) return launch_reg<24, F8>(x, q, scale, R, nchunk, stream);
  const int64_t blocks = (R + kRowsPerBlock - 1) / kRowsPerBlock;
  hipLaunchKernelGGL((quantize_rows_2pass<F8>), dim3((unsigned)blocks), dim3(kThreads), 0, stream,
                     reinterpret_cast<const u32x4*>(x), reinterpret_cast<u32x2*>(q), scale, R,
                     nchunk);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_quantize_rows(const uint16_t* x, int8_t* q, float* scale, int64_t R, int64_t K,
                                hipStream_t stream) {
  return launch_rows<false>(x, q, scale, R, K, stream);
}

hipError_t launch_quantize_rows_fp8(const uint16_t* x, uint8_t* q, float* scale, int64_t R,
                                    int64_t K, hipStream_t stream) {
  return launch_rows<true>(x, reinterpret_cast<int8_t*>(q), scale, R, K, stream);
}

}  // namespace w8a8
