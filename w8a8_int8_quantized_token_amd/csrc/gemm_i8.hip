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
// Pipeline: a workgroup owns a BM x BN output tile and walks K in stages of
// 64 bytes.  Stages go straight from global memory into a ring of S LDS
// buffers with buffer_load ... lds (no staging registers, no LDS store
// instructions); a stage is requested S-1 stages before it is used.  Chunks
// past K or rows past M/N are requested at an out-of-range buffer offset,
// which the hardware returns as zeros, so partial tiles need no branches and
// stages past the end add nothing.  Fragments are read with 16-byte LDS
// reads, one MFMA K step ahead of the MFMAs that use them, including across
// the stage boundary.  16-byte chunks are XOR swizzled within each LDS row so
// that neither the DMA writes nor the fragment reads conflict on banks.  The
// accumulators stay in registers for the whole K loop; int32 never touches
// HBM on the fused path.
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
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;
constexpr int kNumXcd = 8;
constexpr int kGroupM = 4;
constexpr int kDmaBytes = kWave * 16;    // one wavefront DMA: 64 lanes x 16 B
constexpr uint32_t kOOB = 0x80000000u;    // buffer offset beyond any tile: reads as zero
constexpr int kRsrcWord3 = 0x00020000;    // raw buffer, 32-bit data format (gfx9 family)

// S >= 2: ring of S whole stages.  S == 0: split ring -- three X slots and
// two W slots of BM x BK bytes each, so X is requested two stages ahead and
// W one (see the main loop).
template <int BM_, int BN_, int BK_, int WM_, int WN_, int S_>
struct Tile {
  static constexpr int BM = BM_;  // X rows (tokens) per workgroup
  static constexpr int BN = BN_;  // W rows (output channels) per workgroup
  static constexpr int BK = BK_;  // K bytes per stage = bytes per LDS row
  static constexpr int WM = WM_;  // wavefronts along M
  static constexpr int WN = WN_;  // wavefronts along N
  static constexpr bool kSplit = S_ == 0;
  static constexpr int S = kSplit ? 2 : S_;   // whole stages in the ring (split: see above)
  static constexpr int kWaves = WM * WN;
  static constexpr int kThreads = kWaves * kWave;
  static constexpr int TM = BM / WM, TN = BN / WN;   // per-wavefront extent
  static constexpr int FM = TM / 32, FN = TN / 32;   // 32x32 MFMA tiles per wavefront
  static constexpr int KSUB = BK / 32;               // MFMA K steps per stage
  static constexpr int CPR = BK / 16;                // 16-byte chunks per LDS row
  static constexpr int kDmaRows = kDmaBytes / BK;    // rows moved by one wavefront DMA
  static constexpr int DX = BM / kDmaRows / kWaves;  // X DMAs per wavefront per stage
  static constexpr int DW = BN / kDmaRows / kWaves;  // W DMAs per wavefront per stage
  static constexpr int D = DX + DW;
  static constexpr int kStageBytes = (BM + BN) * BK;
  // LDS arrays: split ring -> lds0..2 hold X stages, lds3..4 W stages;
  // otherwise lds0..S-1 hold whole stages.
  static constexpr int kSlots = kSplit ? 5 : S;
  static constexpr int kArr012 = kSplit ? BM * BK : kStageBytes;
  static constexpr int kArr34 = kSplit ? BN * BK : kStageBytes;
  static constexpr int kLdsBytes = kSplit ? 3 * kArr012 + 2 * kArr34 : S * kStageBytes;
  static_assert(BK == 64 || BK == 128, "64- or 128-byte stages");
  static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile must be a multiple of 32");
  static_assert(DX >= 1 && DW >= 1 && DX * kDmaRows * kWaves == BM && DW * kDmaRows * kWaves == BN,
                "every wavefront moves whole DMA blocks of X and W");
  static_assert(S >= 2 && S <= 4, "ring of 2 to 4 stages");
  static_assert((S - 1) * D <= 63, "vmcnt range");
  static_assert(kLdsBytes <= 160 * 1024, "LDS budget");
};

// Physical 16-byte chunk of logical chunk c in LDS row r (CPR chunks per
// row).  gfx950 serves a 16-byte LDS access for 16 lanes at a time out of a
// 256-byte bank window.  Fragment reads take 16 consecutive rows at one chunk
// and a DMA writes 256/(16*CPR) consecutive rows at every chunk; the XOR puts
// both sets into 16 distinct 16-byte slots of the window (measured: reads at
// the linear-access rate, against 1.6x-3x slower without it).
template <int CPR>
__device__ __forceinline__ int swz(int r, int c) {
  if constexpr (CPR == 4) return c ^ ((r >> 2) & 3);
  else return c ^ ((r >> 1) & 7);
}

// One wavefront DMA of 16 bytes per lane from a raw buffer into LDS.  (Kept
// out of the kernel's lambdas: called from a lambda directly, the builtin
// keeps the host pass from emitting the kernel's launch stub.)
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int8_t* lds, uint32_t voffset) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, (int)voffset, 0, 0, 0);
}

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
}

// y = fl32(fl32(fl32(float(acc) * sa) * sw) + b), each step rounded on its own.
__device__ __forceinline__ float dequant(int acc, float sa, float sw, float b) {
  return __fadd_rn(__fmul_rn(__fmul_rn((float)acc, sa), sw), b);
}

// s_waitcnt vmcnt(n) leaving the other counters alone (gfx9 encoding).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
  static_assert(n >= 0 && n < 64, "vmcnt range");
  __builtin_amdgcn_s_waitcnt((n & 0xF) | ((n >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}
__device__ __forceinline__ void wait_lgkmcnt0() { __builtin_amdgcn_s_waitcnt(0xC07F); }

// Workgroup barrier without a memory fence: every wait it relies on is
// issued explicitly before it.
__device__ __forceinline__ void barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

template <class T, Epilogue EPI>
__global__ __launch_bounds__(T::kThreads, 1) void gemm_i8_kernel(
    const int8_t* __restrict__ X, const int8_t* __restrict__ W, const float* __restrict__ sx,
    const float* __restrict__ sw, const uint16_t* __restrict__ bias, void* __restrict__ out,
    int M, int N, int K, int ldy, int tiles_m, int tiles_n, int vec_store) {
  // One array per ring slot: distinct objects let the compiler see that a
  // DMA into one slot never aliases fragment reads from another.
  __shared__ __attribute__((aligned(16))) int8_t lds0[T::kArr012];
  __shared__ __attribute__((aligned(16))) int8_t lds1[T::kArr012];
  __shared__ __attribute__((aligned(16))) int8_t lds2[T::kSlots > 2 ? T::kArr012 : 16];
  __shared__ __attribute__((aligned(16))) int8_t lds3[T::kSlots > 3 ? T::kArr34 : 16];
  __shared__ __attribute__((aligned(16))) int8_t lds4[T::kSlots > 4 ? T::kArr34 : 16];
  int8_t* const ring[4] = {lds0, lds1, lds2, lds3};

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
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / T::WN, wn = wave % T::WN;

  // ---- DMA addressing ----
  // Lane p of a DMA fills LDS slot p of a block of kDmaRows rows (DMA writes
  // are linear, hence conflict-free): row r = block*kDmaRows + p/CPR,
  // physical chunk p%CPR, so the lane fetches logical chunk swz(r, p%CPR).
  const int rows_x = min(T::BM, M - m0), rows_w = min(T::BN, N - n0);
  const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(X + (int64_t)m0 * K), (short)0, rows_x * K, kRsrcWord3);
  const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
      const_cast<int8_t*>(W + (int64_t)n0 * K), (short)0, rows_w * K, kRsrcWord3);
  const int dma_r = lane / T::CPR;
  int xcol[T::DX], wcol[T::DW];        // K byte offset of the lane's chunk in a stage
  uint32_t xrow[T::DX], wrow[T::DW];   // byte offset of that chunk in stage 0, or kOOB
#pragma unroll
  for (int i = 0; i < T::DX; ++i) {
    const int r = (wave + i * T::kWaves) * T::kDmaRows + dma_r;
    xcol[i] = swz<T::CPR>(r, lane % T::CPR) * 16;
    xrow[i] = r < rows_x ? (uint32_t)(r * K + xcol[i]) : kOOB;
  }
#pragma unroll
  for (int i = 0; i < T::DW; ++i) {
    const int r = (wave + i * T::kWaves) * T::kDmaRows + dma_r;
    wcol[i] = swz<T::CPR>(r, lane % T::CPR) * 16;
    wrow[i] = r < rows_w ? (uint32_t)(r * K + wcol[i]) : kOOB;
  }
  // Request the X (W) part of stage kt into `buf`; chunks at or past K read
  // as zeros.
  auto issue_x = [&](int8_t* buf, int kt) {
    const int kb = kt * T::BK;
#pragma unroll
    for (int i = 0; i < T::DX; ++i)
      dma16(rx, buf + (wave + i * T::kWaves) * kDmaBytes,
            kb + xcol[i] < K ? xrow[i] + (uint32_t)kb : kOOB);
  };
  auto issue_w = [&](int8_t* buf, int kt) {
    const int kb = kt * T::BK;
#pragma unroll
    for (int i = 0; i < T::DW; ++i)
      dma16(rw, buf + (wave + i * T::kWaves) * kDmaBytes,
            kb + wcol[i] < K ? wrow[i] + (uint32_t)kb : kOOB);
  };
  // Whole stage kt into ring slot `buf` (X rows first, then W rows).
  auto issue = [&](int8_t* buf, int kt) {
    issue_x(buf, kt);
    issue_w(buf + T::BM * T::BK, kt);
  };

  v16i acc[T::FM][T::FN];
#pragma unroll
  for (int i = 0; i < T::FM; ++i)
#pragma unroll
    for (int j = 0; j < T::FN; ++j) acc[i][j] = v16i{};

  const int row_in = lane % 32;   // row of the 32-row MFMA operand this lane feeds
  const int khalf = lane / 32;    // which 16-byte half of each 32-byte K step

  // The epilogue's scales and bias are requested now, ahead of the stage
  // DMAs, so their latency is hidden by the K loop (the in-order vector memory
  // counter keeps the DMA waits below exact).
  float sa_pre[T::FM], sw_pre = 0.0f, b_pre = 0.0f;
  if constexpr (EPI == Epilogue::kBf16ScaleBias) {
#pragma unroll
    for (int i = 0; i < T::FM; ++i) sa_pre[i] = sx[min(m0 + wm * T::TM + i * 32 + row_in, M - 1)];
    if (tid < T::BN && n0 + tid < N) {
      sw_pre = sw[n0 + tid];
      if (bias != nullptr) b_pre = bf16_to_float(bias[n0 + tid]);
    }
  }

  // Fragment registers, double buffered by MFMA K step parity.
  v4i a[2][T::FN], b[2][T::FM];
  auto frag2 = [&](const int8_t* xs, const int8_t* ws, int s, int slot) {
    const int c = s * 2 + khalf;
#pragma unroll
    for (int j = 0; j < T::FN; ++j) {
      const int r = wn * T::TN + j * 32 + row_in;
      a[slot][j] = *reinterpret_cast<const v4i*>(ws + r * T::BK + swz<T::CPR>(r, c) * 16);
    }
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int r = wm * T::TM + i * 32 + row_in;
      b[slot][i] = *reinterpret_cast<const v4i*>(xs + r * T::BK + swz<T::CPR>(r, c) * 16);
    }
  };
  auto frag = [&](const int8_t* buf, int s, int slot) { frag2(buf, buf + T::BM * T::BK, s, slot); };
  auto mfmas = [&](int slot) {
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j)
        acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(a[slot][j], b[slot][i], acc[i][j], 0, 0, 0);
  };

  // Scheduling of the code after a barrier: the next stage's first fragment
  // reads, then the last K step's MFMAs each followed by one stage request
  // (and its address arithmetic), so the MFMA pipe restarts right away.
  auto interleave = [&]() {
    __builtin_amdgcn_sched_group_barrier(0x100, T::FM + T::FN, 0);   // fragment reads
#pragma unroll
    for (int q = 0; q < T::FM * T::FN; ++q) {
      __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // one MFMA
      __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);             // address VALU
      __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);             // one DMA
    }
    __builtin_amdgcn_sched_barrier(0);
  };

  const int KT = (K + T::BK - 1) / T::BK;
  const int KTr = (KT + T::S - 1) / T::S * T::S;   // stages computed (the extra ones are zeros)

  // Step k (stage k in slot `cur`, fragments of its first K step in flight):
  // run the K steps; once every wavefront is past its reads of `cur` and
  // stage k+1 has landed (one barrier), request stage k+S into `cur` and
  // start reading stage k+1's first fragments under the MFMAs of the last K
  // step.  A stage is thus requested a full S-1 steps before it is needed.
  auto step = [&](int8_t* cur, int8_t* nxt, int k) {
#pragma unroll
    for (int s = 0; s + 1 < T::KSUB; ++s) {
      frag(cur, s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkmcnt0();                 // this wavefront's reads of `cur` are done
    wait_vmcnt<(T::S - 2) * T::D>();  // its DMAs of stage k+1 have landed
    barrier();                       // ... and everyone's
    frag(nxt, 0, T::KSUB & 1);
    issue(cur, k + T::S);
    mfmas((T::KSUB - 1) & 1);
    interleave();
  };

  // Split-ring step k: X_k in `xc`, W_k in `wc`, stage k+1 in `xn`/`wn1`.
  // After the barrier that frees X_k's and W_k's slots, W_{k+2} and then
  // X_{k+3} are requested into them: at the next barrier only the W part
  // (half a stage, requested one step earlier) is on the critical path, while
  // X has two steps to land.
  auto step_split = [&](int8_t* xc, int8_t* wc, int8_t* xn, int8_t* wn1, int k) {
#pragma unroll
    for (int s = 0; s + 1 < T::KSUB; ++s) {
      frag2(xc, wc, s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkmcnt0();
    wait_vmcnt<T::DX>();   // everything but X_{k+2} (the last request) has landed
    barrier();
    // After the barrier: the next stage's first fragment reads, the last K
    // step's MFMAs and the next requests, interleaved so that the MFMA pipe
    // restarts right away instead of waiting for the DMA issue.
    frag2(xn, wn1, 0, T::KSUB & 1);
    issue_w(wc, k + 2);
    issue_x(xc, k + 3);
    mfmas((T::KSUB - 1) & 1);
    interleave();
  };

  // ---- main loop over a ring of S slots ----
  if constexpr (T::kSplit) {
    // X slots lds0..lds2 (X_k in slot k%3), W slots lds3, lds4 (W_k in k%2);
    // the slot pattern repeats every 6 stages.
    issue_x(lds0, 0);
    issue_w(lds3, 0);
    issue_x(lds1, 1);
    issue_w(lds4, 1);
    issue_x(lds2, 2);
    wait_vmcnt<2 * T::DX + T::DW>();
    barrier();
    frag2(lds0, lds3, 0, 0);
    const int KT6 = (KT + 5) / 6 * 6;
    for (int kt = 0; kt < KT6; kt += 6) {
      step_split(lds0, lds3, lds1, lds4, kt);
      step_split(lds1, lds4, lds2, lds3, kt + 1);
      step_split(lds2, lds3, lds0, lds4, kt + 2);
      step_split(lds0, lds4, lds1, lds3, kt + 3);
      step_split(lds1, lds3, lds2, lds4, kt + 4);
      step_split(lds2, lds4, lds0, lds3, kt + 5);
    }
  } else {
#pragma unroll
    for (int s = 0; s < T::S; ++s) issue(ring[s], s);
    wait_vmcnt<(T::S - 1) * T::D>();
    barrier();
    frag(ring[0], 0, 0);
    for (int kt = 0; kt < KTr; kt += T::S) {
      if constexpr (T::S == 2) {
        step(lds0, lds1, kt);
        step(lds1, lds0, kt + 1);
      } else if constexpr (T::S == 3) {
        step(lds0, lds1, kt);
        step(lds1, lds2, kt + 1);
        step(lds2, lds0, kt + 2);
      } else {
        step(lds0, lds1, kt);
        step(lds1, lds2, kt + 1);
        step(lds2, lds3, kt + 2);
        step(lds3, lds0, kt + 3);
      }
    }
  }
  wait_vmcnt<0>();
  wait_lgkmcnt0();
  barrier();   // every DMA and fragment read is done before LDS is reused

  // ---- epilogue: lane holds token m, channels n = base + 8*g + 4*khalf + 0..3 ----
  if constexpr (EPI == Epilogue::kBf16ScaleBias) {
    // The block's channel scales and bias (as fp32) go to LDS once, so each
    // group of 4 outputs needs two 16-byte LDS reads instead of 8 global loads.
    // After the K loop the ring is free: the wavefronts' transpose regions
    // take lds0 (and lds1 if they do not fit), the scales and bias the next
    // array.
    constexpr int RB = T::TN * 2;                          // bytes per region row
    constexpr int kRegion = 32 * RB;                       // 32 rows per wavefront
    constexpr int kPerArr = T::kArr012 / kRegion;          // regions per array
    static_assert(kPerArr >= 1 && (T::kWaves + kPerArr - 1) / kPerArr <= 2, "regions fit in lds0/lds1");
    constexpr bool kOneArr = T::kWaves <= kPerArr;
    int8_t* const sb_arr = kOneArr ? lds1 : lds2;
    static_assert(kOneArr || T::kSlots > 2, "a third array holds the scales");
    float* s_lds = reinterpret_cast<float*>(sb_arr);
    float* b_lds = s_lds + T::BN;
    static_assert(2 * T::BN * 4 <= T::kArr012, "scales and bias fit in one array");
    static_assert(T::BN <= T::kThreads, "one thread per channel of the block");
    if (tid < T::BN) {
      s_lds[tid] = sw_pre;
      b_lds[tid] = b_pre;
    }
    __syncthreads();
    // 4 bf16 outputs (two packed words) of MFMA tile (i, j), run g.
    auto outputs = [&](int i, int j, int g, float sa, uint32_t& wlo, uint32_t& whi) {
      const int nl = wn * T::TN + j * 32 + g * 8 + khalf * 4;
      const f32x4 sv = *reinterpret_cast<const f32x4*>(s_lds + nl);
      const f32x4 bv = *reinterpret_cast<const f32x4*>(b_lds + nl);
      const v16i& c = acc[i][j];
      const bf16x2 lo = __builtin_convertvector(
          (f32x2{dequant(c[g * 4], sa, sv[0], bv[0]), dequant(c[g * 4 + 1], sa, sv[1], bv[1])}), bf16x2);
      const bf16x2 hi = __builtin_convertvector(
          (f32x2{dequant(c[g * 4 + 2], sa, sv[2], bv[2]), dequant(c[g * 4 + 3], sa, sv[3], bv[3])}), bf16x2);
      wlo = __builtin_bit_cast(uint32_t, lo);
      whi = __builtin_bit_cast(uint32_t, hi);
    };
    if (vec_store) {
      // Row-major Y with N % 8 == 0: each wavefront turns 32 rows x TN of its
      // results around in its own LDS region and writes whole 16-byte row
      // chunks, so a store instruction covers full 128-byte lines instead of
      // 32 scattered 16-byte pieces.
      constexpr int RCH = RB / 16;                    // 16-byte chunks per region row
      constexpr bool kPow2 = (RCH & (RCH - 1)) == 0;
      constexpr int RWIN = RB >= 256 ? 1 : 256 / RB;  // region rows per 256-byte bank window
      constexpr int RPI = kWave / RCH;                // rows per wavefront store
      constexpr int NIT = (32 + RPI - 1) / RPI;       // stores per 32 rows
      int8_t* region = (wave < kPerArr ? lds0 + wave * kRegion : lds1 + (wave - kPerArr) * kRegion);
      // XOR swizzle of the 16-byte chunks for power-of-two row widths (the
      // 96-channel rows of 192-wide tiles are read linearly instead)
      auto rsw = [](int r, int c) { return kPow2 ? (c ^ ((r / RWIN) & (RCH - 1))) : c; };
      const int n = n0 + wn * T::TN + (lane % RCH) * 8;   // this lane's 8 channels when storing
      const bool lane_on = lane < RPI * RCH;
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        const int mb = m0 + wm * T::TM + i * 32;
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint32_t wlo, whi;
            outputs(i, j, g, sa_pre[i], wlo, whi);
            *reinterpret_cast<u32x2*>(region + row_in * RB + rsw(row_in, 4 * j + g) * 16 + 8 * khalf) =
                u32x2{wlo, whi};
          }
        }
        v4i v[NIT];
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int r = min(it * RPI + lane / RCH, 31);
          v[it] = *reinterpret_cast<const v4i*>(region + r * RB + rsw(r, lane % RCH) * 16);
        }
#pragma unroll
        for (int it = 0; it < NIT; ++it) {
          const int r = it * RPI + lane / RCH;
          const int m = mb + r;
          if (lane_on && r < 32 && m < M && n < N)
            *reinterpret_cast<v4i*>(reinterpret_cast<uint16_t*>(out) + (int64_t)m * ldy + n) = v[it];
        }
      }
    } else {
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        const int m = m0 + wm * T::TM + i * 32 + row_in;
        if (m >= M) continue;
        uint16_t* yrow = reinterpret_cast<uint16_t*>(out) + (int64_t)m * ldy;
        const float sa = sa_pre[i];
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            uint32_t wlo, whi;
            outputs(i, j, g, sa, wlo, whi);
            const int n = n0 + wn * T::TN + j * 32 + g * 8 + khalf * 4;
            const uint16_t h[4] = {(uint16_t)wlo, (uint16_t)(wlo >> 16), (uint16_t)whi,
                                   (uint16_t)(whi >> 16)};
#pragma unroll
            for (int e = 0; e < 4; ++e)
              if (n + e < N) yrow[n + e] = h[e];
          }
        }
      }
    }
  } else {
#pragma unroll
    for (int i = 0; i < T::FM; ++i) {
      const int m = m0 + wm * T::TM + i * 32 + row_in;
      if (m >= M) continue;
      int32_t* crow = reinterpret_cast<int32_t*>(out) + (int64_t)m * ldy;
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

// Launch tile configuration T on the sub-problem M x N x K whose output rows
// are `ldy` elements apart.
template <class T>
hipError_t launch_t(Epilogue epi, const int8_t* xq, const int8_t* wq, const float* sx,
                    const float* sw, const uint16_t* bias, void* out, int64_t M, int64_t N,
                    int64_t K, int64_t ldy, hipStream_t stream) {
  const int tiles_m = (int)((M + T::BM - 1) / T::BM);
  const int tiles_n = (int)((N + T::BN - 1) / T::BN);
  const dim3 grid((unsigned)(tiles_m * tiles_n));
  const dim3 block(T::kThreads);
  const uintptr_t o = reinterpret_cast<uintptr_t>(out);
  if (epi == Epilogue::kBf16ScaleBias) {
    const int vec = (ldy % 8 == 0) && (o % 16 == 0);
    hipLaunchKernelGGL((gemm_i8_kernel<T, Epilogue::kBf16ScaleBias>), grid, block, 0, stream, xq,
                       wq, sx, sw, bias, out, (int)M, (int)N, (int)K, (int)ldy, tiles_m, tiles_n,
                       vec);
  } else {
    const int vec = (ldy % 4 == 0) && (o % 16 == 0);
    hipLaunchKernelGGL((gemm_i8_kernel<T, Epilogue::kRawI32>), grid, block, 0, stream, xq, wq,
                       nullptr, nullptr, nullptr, out, (int)M, (int)N, (int)K, (int)ldy, tiles_m,
                       tiles_n, vec);
  }
  return hipGetLastError();
}

// Compiled tile configurations.
using CfgSplit = Tile<256, 256, 128, 2, 4, 0>;   // 256x256, X two stages ahead, W one
using CfgWhole = Tile<256, 256, 128, 2, 4, 2>;   // 256x256, two whole stages
using Cfg192 = Tile<256, 192, 128, 4, 2, 0>;     // 256x192, split ring
using CfgTail = Tile<128, 256, 128, 2, 4, 3>;    // 128x256, three whole stages
using Cfg256x128 = Tile<256, 128, 128, 2, 2, 3>;
using Cfg128 = Tile<128, 128, 64, 2, 2, 4>;
using Cfg64 = Tile<64, 64, 64, 2, 2, 3>;

template <class T>
constexpr TileDesc desc() { return TileDesc{T::BM, T::BN, T::BK, T::kThreads}; }

enum Cfg { kSplit256, kWhole256, k192, kTail128x256, k256x128, k128, k64, kNumCfg };
const TileDesc kCfgs[kNumCfg] = {desc<CfgSplit>(), desc<CfgWhole>(), desc<Cfg192>(),
                                 desc<CfgTail>(), desc<Cfg256x128>(), desc<Cfg128>(),
                                 desc<Cfg64>()};

hipError_t launch_cfg(int cfg, Epilogue epi, const int8_t* xq, const int8_t* wq, const float* sx,
                      const float* sw, const uint16_t* bias, void* out, int64_t M, int64_t N,
                      int64_t K, int64_t ldy, hipStream_t s) {
  switch (cfg) {
    case kSplit256: return launch_t<CfgSplit>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s);
    case kWhole256: return launch_t<CfgWhole>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s);
    case k192: return launch_t<Cfg192>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s);
    case kTail128x256: return launch_t<CfgTail>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s);
    case k256x128: return launch_t<Cfg256x128>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s);
    case k128: return launch_t<Cfg128>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s);
    case k64: return launch_t<Cfg64>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s);
    default: return hipErrorInvalidValue;
  }
}

// A plan ("tile id" of the C ABI) is a main configuration, optionally with
// a tail: when the main tiles do not come out as whole waves of 256
// workgroups (one per CU), the leading output-channel columns that do are
// done with the main tiles and the remaining columns with 128x256 tiles in a
// second launch, so the last wave of big tiles does not run on a
// half-empty GPU.
struct Plan {
  int main;
  int tail;   // -1: none
};
constexpr Plan kPlans[] = {
    {kSplit256, kTail128x256}, {kSplit256, -1}, {kWhole256, kTail128x256}, {kWhole256, -1},
    {k192, -1}, {kTail128x256, -1}, {k256x128, -1}, {k128, -1}, {k64, -1}};
constexpr int kNumPlans = sizeof(kPlans) / sizeof(kPlans[0]);
constexpr int kCUs = 256;

// Leading columns of main tiles that form whole waves (0: no useful split).
int64_t main_columns(const TileDesc& d, int64_t M, int64_t N) {
  const int64_t tm = (M + d.block_m - 1) / d.block_m, tn = (N + d.block_n - 1) / d.block_n;
  if ((tm * tn) % kCUs == 0) return 0;
  const int64_t rounds = (tm * tn + kCUs - 1) / kCUs;
  const TileDesc& t = kCfgs[kTail128x256];
  for (int64_t c = tn - 1; c >= 1; --c) {
    if ((tm * c) % kCUs != 0) continue;
    const int64_t tail = ((M + t.block_m - 1) / t.block_m) *
                         ((N - c * d.block_n + t.block_n - 1) / t.block_n);
    // a tail wave of half-height tiles costs about 0.6 of a wave of main tiles
    const double est = (double)(tm * c / kCUs) + 0.6 * (double)((tail + kCUs - 1) / kCUs);
    return est + 0.1 < (double)rounds ? c : 0;
  }
  return 0;
}

}  // namespace

int num_tiles() { return kNumPlans; }
const TileDesc& tile_desc(int tile) { return kCfgs[kPlans[tile].main]; }

// Shape -> plan, from sweeps over the DiT shapes on MI355X: 256x256 tiles with
// 128-byte stages (plus the 128x256 tail) whenever they give every CU at least
// one tile -- the split ring when K is a multiple of 6 stages or close enough
// that its zero-padded stages cost < 5%; below that, 256x128, then 128x128,
// then 64x64 tiles keep the 256 CUs busy.
int select_tile(int64_t M, int64_t N, int64_t K) {
  auto tiles = [&](int cfg) {
    return ((M + kCfgs[cfg].block_m - 1) / kCfgs[cfg].block_m) *
           ((N + kCfgs[cfg].block_n - 1) / kCfgs[cfg].block_n);
  };
  if (tiles(kSplit256) >= kCUs) {
    const int64_t kt = (K + 127) / 128;
    const int64_t kt6 = (kt + 5) / 6 * 6;
    return (kt6 - kt) * 20 <= kt ? 0 : 2;
  }
  if (tiles(k256x128) >= kCUs / 2) return 6;
  if (tiles(k128) >= kCUs / 2) return 7;
  return 8;
}

hipError_t launch_gemm(int tile, Epilogue epi, const int8_t* xq, const int8_t* wq,
                       const float* sx, const float* sw, const uint16_t* bias, void* out,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (tile < 0 || tile >= kNumPlans) return hipErrorInvalidValue;
  const Plan& p = kPlans[tile];
  const int64_t c = p.tail >= 0 ? main_columns(kCfgs[p.main], M, N) : 0;
  if (c == 0) return launch_cfg(p.main, epi, xq, wq, sx, sw, bias, out, M, N, K, N, stream);
  const int64_t nm = c * kCfgs[p.main].block_n;   // channels done by the main tiles
  hipError_t e = launch_cfg(p.main, epi, xq, wq, sx, sw, bias, out, M, nm, K, N, stream);
  if (e != hipSuccess) return e;
  const size_t esz = epi == Epilogue::kBf16ScaleBias ? 2 : 4;
  void* out_tail = static_cast<char*>(out) + nm * esz;
  return launch_cfg(p.tail, epi, xq, wq + nm * K, sx, sw ? sw + nm : nullptr,
                    bias ? bias + nm : nullptr, out_tail, M, N - nm, K, N, stream);
}

}  // namespace w8a8
