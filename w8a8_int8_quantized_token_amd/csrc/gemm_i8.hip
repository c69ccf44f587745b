// int8 x int8 -> int32 GEMM on gfx950 matrix cores with a fused per-token x
// per-channel dequant + bias epilogue that writes bf16 (or, for the
// diagnostic entry, the raw int32 accumulators).  This is the fused kernel
// of the abstract of "Realizing Native INT8 Compute for Diffusion
// Transformers on Consumer GPUs" (arXiv 2606.14598), designed for CDNA4.
//
// Operands: X = xq [M,K] (tokens) and W = wq [N,K] (output channels), both
// K-contiguous, which is exactly the per-lane operand layout of
// v_mfma_i32_32x32x32_i8 (each lane supplies 16 consecutive K bytes of one
// row).  The MFMA's first operand takes W rows and its second X rows, so the
// 32x32 result a lane holds is one token (column) by 16 output channels in
// four runs of 4 consecutive channels: the epilogue writes 8-byte runs of a
// row of Y without any transpose.
//
// Pipeline: a workgroup owns a BM x BN output tile; K is walked in stages of
// BK bytes.  Each stage of X and W is fetched with 16-byte global loads into
// registers, written to one of two LDS buffers (double buffering: the next
// stage's global loads are in flight while the current stage feeds the
// MFMAs), and read back with 16-byte LDS reads.  16-byte chunks are XOR
// swizzled within each LDS row so that the 32 rows a wavefront reads at one
// K offset fall in distinct banks.  The accumulators (FM x FN tiles of 16
// int32 per lane) stay in registers for the whole K loop; int32 never
// touches HBM on the fused path.
//
// Workgroup order: consecutive workgroup ids are dispatched round robin over
// the 8 XCDs, each with its own L2.  Ids are remapped so that each XCD gets a
// contiguous range of tiles, and that range is walked in groups of kGroupM
// tile rows, so the tiles resident on one XCD share X and W panels in its L2.
#include "kernels.h"

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kWave = 64;
constexpr int kNumXcd = 8;
constexpr int kGroupM = 4;

template <int BM_, int BN_, int BK_, int WM_, int WN_>
struct Tile {
  static constexpr int BM = BM_;  // X rows (tokens) per workgroup
  static constexpr int BN = BN_;  // W rows (output channels) per workgroup
  static constexpr int BK = BK_;  // K bytes per stage
  static constexpr int WM = WM_;  // wavefronts along M
  static constexpr int WN = WN_;  // wavefronts along N
  static constexpr int kThreads = WM * WN * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;   // per-wavefront extent
  static constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 MFMA tiles per wavefront
  static constexpr int CPR = BK / 16;                // 16-byte chunks per LDS row
  static constexpr int XCH = BM * CPR / kThreads;    // X chunks per thread per stage
  static constexpr int WCH = BN * CPR / kThreads;    // W chunks per thread per stage
  static constexpr int RSTEP = kThreads / CPR;       // rows between a thread's chunks
  static constexpr int kStageBytes = (BM + BN) * BK;
  static constexpr int kLdsBytes = 2 * kStageBytes;
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(BK % 32 == 0 && CPR >= 2 && CPR <= 8, "BK must be 32..128");
  static_assert(kThreads % CPR == 0, "threads must cover whole rows");
  static_assert(XCH * kThreads == BM * CPR && WCH * kThreads == BN * CPR, "uneven chunk split");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// Physical 16-byte chunk of logical chunk c in LDS row r.
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  return c ^ (r & (CPR - 1));
}

__device__ __forceinline__ uint32_t bf16_rne_bits(float f) {
  uint32_t u = __float_as_uint(f);
  return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;  // finite inputs
}

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// y = fl32(fl32(fl32(float(acc) * sa) * sw) + b), each step rounded on its own.
__device__ __forceinline__ float dequant(int acc, float sa, float sw, float b) {
  return __fadd_rn(__fmul_rn(__fmul_rn((float)acc, sa), sw), b);
}

template <class T, Epilogue EPI>
__global__ __launch_bounds__(T::kThreads, 1) void gemm_i8_kernel(
    const int8_t* __restrict__ X, const int8_t* __restrict__ W, const float* __restrict__ sx,
    const float* __restrict__ sw, const uint16_t* __restrict__ bias, void* __restrict__ out,
    int M, int N, int K, int tiles_m, int tiles_n, int vec_store) {
  __shared__ __attribute__((aligned(16))) int8_t lds[T::kLdsBytes];

  // ---- workgroup -> output tile (XCD-aware, grouped along M) ----
  const int ntiles = tiles_m * tiles_n;
  int bid = blockIdx.x;
  if (ntiles % kNumXcd == 0) bid = (bid % kNumXcd) * (ntiles / kNumXcd) + bid / kNumXcd;
  const int per_group = kGroupM * tiles_n;
  const int group = bid / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = bid - group * per_group;
  const int tm = first_m + in_group % gsize;
  const int tn = in_group / gsize;
  const int m0 = tm * T::BM, n0 = tn * T::BN;

  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = tid / kWave;
  const int wm = wave / T::WN, wn = wave % T::WN;

  // ---- global -> register staging addresses (32-bit offsets in the tile) ----
  const int ld_c = tid % T::CPR;    // chunk column, the same for all of a thread's chunks
  const int ld_r = tid / T::CPR;    // first row
  const int8_t* xblk = X + (int64_t)m0 * K;
  const int8_t* wblk = W + (int64_t)n0 * K;
  int xoff[T::XCH], woff[T::WCH];
#pragma unroll
  for (int i = 0; i < T::XCH; ++i) {
    const int r = ld_r + i * T::RSTEP;
    xoff[i] = (min(m0 + r, M - 1) - m0) * K + ld_c * 16;   // rows past M re-read row M-1
  }
#pragma unroll
  for (int i = 0; i < T::WCH; ++i) {
    const int r = ld_r + i * T::RSTEP;
    woff[i] = (min(n0 + r, N - 1) - n0) * K + ld_c * 16;
  }
  v4i xreg[T::XCH], wreg[T::WCH];

  auto load_stage = [&](int kt) {
    const int kb = kt * T::BK;
    const bool ok = kb + ld_c * 16 < K;   // K % 16 == 0: a chunk is all in or all out
#pragma unroll
    for (int i = 0; i < T::XCH; ++i)
      xreg[i] = ok ? *reinterpret_cast<const v4i*>(xblk + xoff[i] + kb) : v4i{0, 0, 0, 0};
#pragma unroll
    for (int i = 0; i < T::WCH; ++i)
      wreg[i] = ok ? *reinterpret_cast<const v4i*>(wblk + woff[i] + kb) : v4i{0, 0, 0, 0};
  };
  auto store_stage = [&](int buf) {
    int8_t* xs = lds + buf * T::kStageBytes;
    int8_t* ws = xs + T::BM * T::BK;
#pragma unroll
    for (int i = 0; i < T::XCH; ++i) {
      const int r = ld_r + i * T::RSTEP;
      *reinterpret_cast<v4i*>(xs + r * T::BK + swz<T::CPR>(r, ld_c) * 16) = xreg[i];
    }
#pragma unroll
    for (int i = 0; i < T::WCH; ++i) {
      const int r = ld_r + i * T::RSTEP;
      *reinterpret_cast<v4i*>(ws + r * T::BK + swz<T::CPR>(r, ld_c) * 16) = wreg[i];
    }
  };

  v16i acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = v16i{};

  const int row_in = lane % 32;   // row of the 32-row MFMA operand this lane feeds
  const int khalf = lane / 32;    // which 16-byte half of each 32-byte K step
  const int KT = (K + T::BK - 1) / T::BK;

  load_stage(0);
  store_stage(0);
  __syncthreads();
  for (int kt = 0; kt < KT; ++kt) {
    const bool more = kt + 1 < KT;
    if (more) load_stage(kt + 1);
    const int8_t* xs = lds + (kt & 1) * T::kStageBytes;
    const int8_t* ws = xs + T::BM * T::BK;
#pragma unroll
    for (int kk = 0; kk < T::BK / 32; ++kk) {
      const int c = kk * 2 + khalf;
      v4i a[T::FN], b[T::FM];
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        const int r = wn * T::TN + j * 32 + row_in;
        a[j] = *reinterpret_cast<const v4i*>(ws + r * T::BK + swz<T::CPR>(r, c) * 16);
      }
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        const int r = wm * T::TM + i * 32 + row_in;
        b[i] = *reinterpret_cast<const v4i*>(xs + r * T::BK + swz<T::CPR>(r, c) * 16);
      }
#pragma unroll
      for (int i = 0; i < T::FM; ++i)
#pragma unroll
        for (int j = 0; j < T::FN; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[j], b[i], acc[i][j], 0, 0, 0);
    }
    if (more) store_stage((kt + 1) & 1);
    __syncthreads();
  }

  // ---- epilogue: lane holds token m, channels n = base + 8*g + 4*khalf + 0..3 ----
#pragma unroll
  for (int i = 0; i < T::FM; ++i) {
    const int m = m0 + wm * T::TM + i * 32 + row_in;
    if (m >= M) continue;
    if constexpr (EPI == Epilogue::kBf16ScaleBias) {
      uint16_t* yrow = reinterpret_cast<uint16_t*>(out) + (int64_t)m * N;
      const float sa = sx[m];
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * T::TN + j * 32 + g * 8 + khalf * 4;
          if (vec_store && n + 3 < N) {
            uint32_t h[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              const float b = bias ? bf16_to_float(bias[n + e]) : 0.0f;
              h[e] = bf16_rne_bits(dequant(acc[i][j][g * 4 + e], sa, sw[n + e], b));
            }
            *reinterpret_cast<u32x2*>(yrow + n) = u32x2{h[0] | (h[1] << 16), h[2] | (h[3] << 16)};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              if (n + e < N) {
                const float b = bias ? bf16_to_float(bias[n + e]) : 0.0f;
                yrow[n + e] = (uint16_t)bf16_rne_bits(dequant(acc[i][j][g * 4 + e], sa, sw[n + e], b));
              }
            }
          }
        }
      }
    } else {
      int32_t* crow = reinterpret_cast<int32_t*>(out) + (int64_t)m * N;
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const int n = n0 + wn * T::TN + j * 32 + g * 8 + khalf * 4;
          if (vec_store && n + 3 < N) {
            *reinterpret_cast<v4i*>(crow + n) =
                v4i{acc[i][j][g * 4], acc[i][j][g * 4 + 1], acc[i][j][g * 4 + 2], acc[i][j][g * 4 + 3]};
          } else {
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) crow[n + e] = acc[i][j][g * 4 + e];
          }
        }
      }
    }
  }
}

template <class T>
hipError_t launch_t(Epilogue epi, const int8_t* xq, const int8_t* wq, const float* sx,
                    const float* sw, const uint16_t* bias, void* out, int64_t M, int64_t N,
                    int64_t K, hipStream_t stream) {
  const int tiles_m = (int)((M + T::BM - 1) / T::BM);
  const int tiles_n = (int)((N + T::BN - 1) / T::BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  const dim3 block(T::kThreads);
  const uintptr_t o = reinterpret_cast<uintptr_t>(out);
  if (epi == Epilogue::kBf16ScaleBias) {
    const int vec = (N % 4 == 0) && (o % 8 == 0);
    hipLaunchKernelGGL((gemm_i8_kernel<T, Epilogue::kBf16ScaleBias>), grid, block, 0, stream, xq,
                       wq, sx, sw, bias, out, (int)M, (int)N, (int)K, tiles_m, tiles_n, vec);
  } else {
    const int vec = (N % 4 == 0) && (o % 16 == 0);
    hipLaunchKernelGGL((gemm_i8_kernel<T, Epilogue::kRawI32>), grid, block, 0, stream, xq, wq,
                       nullptr, nullptr, nullptr, out, (int)M, (int)N, (int)K, tiles_m, tiles_n,
                       vec);
  }
  return hipGetLastError();
}

using T0 = Tile<256, 256, 64, 2, 2>;
using T1 = Tile<256, 128, 64, 2, 2>;
using T2 = Tile<128, 256, 64, 2, 2>;
using T3 = Tile<128, 128, 64, 2, 2>;
using T4 = Tile<64, 64, 64, 2, 2>;
using T5 = Tile<256, 256, 128, 2, 2>;

template <class T>
constexpr TileDesc desc() { return TileDesc{T::BM, T::BN, T::BK, T::kThreads}; }

const TileDesc kTiles[] = {desc<T0>(), desc<T1>(), desc<T2>(), desc<T3>(), desc<T4>(), desc<T5>()};
constexpr int kNumTiles = sizeof(kTiles) / sizeof(kTiles[0]);

}  // namespace

int num_tiles() { return kNumTiles; }
const TileDesc& tile_desc(int tile) { return kTiles[tile]; }

// Shape -> tile.  Prefer the largest tile that still gives every CU work.
int select_tile(int64_t M, int64_t N, int64_t K) {
  (void)K;
  const int64_t cus = 256;
  auto tiles = [&](int t) {
    return ((M + kTiles[t].block_m - 1) / kTiles[t].block_m) *
           ((N + kTiles[t].block_n - 1) / kTiles[t].block_n);
  };
  if (tiles(0) >= 4 * cus) return 0;
  if (tiles(1) >= 2 * cus) return 1;
  if (tiles(3) >= cus) return 3;
  return 4;
}

hipError_t launch_gemm(int tile, Epilogue epi, const int8_t* xq, const int8_t* wq,
                       const float* sx, const float* sw, const uint16_t* bias, void* out,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  switch (tile) {
    case 0: return launch_t<T0>(epi, xq, wq, sx, sw, bias, out, M, N, K, stream);
    case 1: return launch_t<T1>(epi, xq, wq, sx, sw, bias, out, M, N, K, stream);
    case 2: return launch_t<T2>(epi, xq, wq, sx, sw, bias, out, M, N, K, stream);
    case 3: return launch_t<T3>(epi, xq, wq, sx, sw, bias, out, M, N, K, stream);
    case 4: return launch_t<T4>(epi, xq, wq, sx, sw, bias, out, M, N, K, stream);
    case 5: return launch_t<T5>(epi, xq, wq, sx, sw, bias, out, M, N, K, stream);
    default: return hipErrorInvalidValue;
  }
}

}  // namespace w8a8
