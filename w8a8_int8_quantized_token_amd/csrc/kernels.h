// Internal launch interface between the C-ABI layer and the HIP kernels of
// libw8a8 (gfx950).  Not installed; the public ABI is include/w8a8.h.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace w8a8 {

// Row-wise absmax quantizer: rows of x [R,K] (bf16 bits) -> q int8 [R,K] and
// scale fp32 [R].  Requires K % 16 == 0 and R > 0.
hipError_t launch_quantize_rows(const uint16_t* x, int8_t* q, float* scale,
                                int64_t R, int64_t K, hipStream_t stream);

// The same with e4m3 codes: scale fl32(amax/448), q = e4m3(fl32(x/scale)).
hipError_t launch_quantize_rows_fp8(const uint16_t* x, uint8_t* q, float* scale, int64_t R,
                                    int64_t K, hipStream_t stream);

// Row-wise dequantization: out[r,k] = bf16(fl32(float(q[r,k]) * scale[r])),
// q int8 [R,K] -> out bf16 bits [R,K].  Requires K % 16 == 0 and R > 0.
hipError_t launch_dequantize_rows(const int8_t* q, const float* scale, uint16_t* out, int64_t R,
                                  int64_t K, hipStream_t stream);

// One compiled GEMM tile configuration.
struct TileDesc {
  int block_m;   // rows of X (tokens) per workgroup
  int block_n;   // rows of W (output channels) per workgroup
  int block_k;   // K bytes staged per pipeline step
  int threads;   // workgroup size
};

int num_tiles();
const TileDesc& tile_desc(int tile);
int select_tile(int64_t M, int64_t N, int64_t K);
// K ranges (1 = no split) and plan the split cost model picks for a shape.
int select_splitk(int64_t M, int64_t N, int64_t K, int* tile);

// kBf16ScaleBias: y = bf16(((acc*sx)*sw)+b); kBf16GeluScaleBias: the same
// value through GELU before the bf16 rounding; kRawI32: the accumulators.
enum class Epilogue { kBf16ScaleBias, kBf16GeluScaleBias, kRawI32 };

// int8 GEMM acc[m,n] = sum_k xq[m,k] * wq[n,k] with the chosen epilogue.
// For the bf16 epilogues `out` is bf16 [M,N] and sx/sw/bias are used (bias
// may be null); for kRawI32 `out` is int32 [M,N].  Shapes already validated.
hipError_t launch_gemm(int tile, Epilogue epi, const int8_t* xq, const int8_t* wq,
                       const float* sx, const float* sw, const uint16_t* bias, void* out,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream);

// K-split int8 GEMM: the main tiles of plan `tile` over `chunks` equal K
// ranges (K % (16 * chunks) == 0), each range's raw int32 sums into its own
// slice partials[c * M * N + m * N + n] (exact; the slices add up to acc).
hipError_t launch_gemm_partials(int tile, const int8_t* xq, const int8_t* wq, int32_t* partials,
                                int64_t M, int64_t N, int64_t K, int chunks, hipStream_t stream);

// Sum of the K-split slices plus the bf16 epilogue (kBf16ScaleBias or
// kBf16GeluScaleBias): y[m,n] from acc = sum_c partials[c][m][n], exactly as
// the fused GEMM's epilogue evaluates it.  Requires N % 8 == 0.
hipError_t launch_splitk_reduce(Epilogue epi, const int32_t* partials, int chunks, const float* sx,
                                const float* sw, const uint16_t* bias, uint16_t* y, int64_t M,
                                int64_t N, hipStream_t stream);

// The fp8 (e4m3) variant: the same tiles and epilogues on
// v_mfma_f32_32x32x64_f8f6f4; for kRawI32 `out` receives the fp32
// accumulators' bits.
hipError_t launch_gemm_fp8(int tile, Epilogue epi, const uint8_t* xq, const uint8_t* wq,
                           const float* sx, const float* sw, const uint16_t* bias, void* out,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream);

// Diagnostic: the fused GEMM's K-step (256x192 tile, eight wavefronts) looped
// `iters` times over one LDS-resident K stage of xq [M,K] and wq [N,K] per
// workgroup, with no memory traffic in the loop; sink int64
// [kCeilingWorkgroups * 8] receives each wavefront's accumulator sum.
// Requires M >= 256, N >= 192, K >= 128 (shapes already validated).
constexpr int kCeilingWorkgroups = 256;
hipError_t launch_mfma_ceiling(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                               int64_t iters, int64_t* sink, hipStream_t stream);

}  // namespace w8a8
