// Diagnostic: the throughput ceiling of the fused GEMM's inner loop on this
// GPU, on the caller's own int8 codes.
//
// The int8 matrix cores of an MI355X run at a power-limited clock whose level
// depends on the operand values (all-zero operands run at the full 2.4 GHz,
// quantized activations and weights far lower).  To put the GEMM's rate
// against what the matrix cores can sustain on the same data, this kernel runs
// the GEMM's K-step exactly -- the 256x192 tile's eight wavefronts of 64x96
// outputs, 16-byte fragment reads from XOR-swizzled LDS one K step ahead of the
// v_mfma_i32_32x32x32_i8 that use them -- but with nothing else: one 128-byte K
// stage of X and W rows is staged in LDS once, and the wavefronts loop over its
// four K steps `iters` times, with no stage requests, no barriers and no
// epilogue.  Its rate is the GEMM's upper bound on this chip for these codes.
//
// Result: every wavefront writes the sum of its int32 accumulators (as int64)
// to sink[workgroup * 8 + wavefront]; over a workgroup these sum to
// iters * sum_k (sum_m x[m,k]) * (sum_n w[n,k]) over the workgroup's rows and
// its K stage, which a test can check exactly.
#include "kernels.h"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));

constexpr int kWave = 64;
constexpr int kBM = 256, kBN = 192, kBK = 128;   // the GEMM's 256x192 tile and stage
constexpr int kWM = 4, kWN = 2;                   // wavefronts along M and N
constexpr int kTM = kBM / kWM, kTN = kBN / kWN;   // 64 x 96 outputs per wavefront
constexpr int kFM = kTM / 32, kFN = kTN / 32;     // 2 x 3 MFMA tiles per wavefront
constexpr int kCPR = kBK / 16;                    // 16-byte chunks per LDS row
constexpr int kThreads = kWM * kWN * kWave;       // 512

// the GEMM's LDS swizzle for 128-byte rows: chunk c of row r at c ^ ((r>>1)&7)
__device__ __forceinline__ int swz(int r, int c) { return c ^ ((r >> 1) & 7); }

__global__ __launch_bounds__(kThreads, 1) void mfma_ceiling_kernel(
    const int8_t* __restrict__ X, const int8_t* __restrict__ W, int M, int N, int K,
    long long iters, long long* __restrict__ sink) {
  __shared__ __attribute__((aligned(16))) int8_t xs[kBM * kBK];
  __shared__ __attribute__((aligned(16))) int8_t ws[kBN * kBK];
  const int tm = M / kBM, tn = N / kBN, tk = K / kBK;   // each >= 1 (checked by the host)
  const int m0 = (int)(blockIdx.x % tm) * kBM;
  const int n0 = (int)((blockIdx.x / tm) % tn) * kBN;
  const int k0 = (int)(blockIdx.x % tk) * kBK;
  for (int i = threadIdx.x; i < kBM * kCPR; i += kThreads) {
    const int r = i / kCPR, c = i % kCPR;
    *reinterpret_cast<v4i*>(xs + r * kBK + swz(r, c) * 16) =
        *reinterpret_cast<const v4i*>(X + (int64_t)(m0 + r) * K + k0 + c * 16);
  }
  for (int i = threadIdx.x; i < kBN * kCPR; i += kThreads) {
    const int r = i / kCPR, c = i % kCPR;
    *reinterpret_cast<v4i*>(ws + r * kBK + swz(r, c) * 16) =
        *reinterpret_cast<const v4i*>(W + (int64_t)(n0 + r) * K + k0 + c * 16);
  }
  __syncthreads();

  const int lane = threadIdx.x % kWave, wave = threadIdx.x / kWave;
  const int wm = wave / kWN, wn = wave % kWN;
  const int row_in = lane % 32, khalf = lane / 32;
  v16i acc[kFM][kFN];
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j) acc[i][j] = v16i{};
  v4i fa[2][kFN], fb[2][kFM];
  // fragments of K step s (0..3) into buffer `slot`: lane half h reads chunk 2s + h
  auto frag = [&](int s, int slot) {
    const int c = s * 2 + khalf;
#pragma unroll
    for (int j = 0; j < kFN; ++j) {
      const int r = wn * kTN + j * 32 + row_in;
      fa[slot][j] = *reinterpret_cast<const v4i*>(ws + r * kBK + swz(r, c) * 16);
    }
#pragma unroll
    for (int i = 0; i < kFM; ++i) {
      const int r = wm * kTM + i * 32 + row_in;
      fb[slot][i] = *reinterpret_cast<const v4i*>(xs + r * kBK + swz(r, c) * 16);
    }
  };
  frag(0, 0);
  for (long long it = 0; it < iters; ++it) {
#pragma unroll
    for (int s = 0; s < 4; ++s) {
      // the LDS stage never changes, so without this the compiler would hoist
      // every fragment read out of the loop; the GEMM re-reads them each step
      asm volatile("" ::: "memory");
      frag((s + 1) & 3, (s + 1) & 1);   // the next K step's fragments, under this step's MFMAs
      __builtin_amdgcn_sched_barrier(0);   // issued before them, as in the GEMM
#pragma unroll
      for (int i = 0; i < kFM; ++i)
#pragma unroll
        for (int j = 0; j < kFN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[s & 1][j], fb[s & 1][i], acc[i][j], 0, 0, 0);
      __builtin_amdgcn_sched_barrier(0);
    }
  }
  long long sum = 0;
#pragma unroll
  for (int i = 0; i < kFM; ++i)
#pragma unroll
    for (int j = 0; j < kFN; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) sum += acc[i][j][e];
#pragma unroll
  for (int off = kWave / 2; off > 0; off >>= 1) sum += __shfl_xor(sum, off, kWave);
  if (lane == 0) sink[(int64_t)blockIdx.x * (kWM * kWN) + wave] = sum;
}

}  // namespace

hipError_t launch_mfma_ceiling(const int8_t* xq, const int8_t* wq, int64_t M, int64_t N, int64_t K,
                               int64_t iters, int64_t* sink, hipStream_t stream) {
  hipLaunchKernelGGL(mfma_ceiling_kernel, dim3(kCeilingWorkgroups), dim3(kThreads), 0, stream, xq, wq,
                     (int)M, (int)N, (int)K, (long long)iters, reinterpret_cast<long long*>(sink));
  return hipGetLastError();
}

}  // namespace w8a8
