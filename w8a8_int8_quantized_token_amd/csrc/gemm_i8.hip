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
// four runs of 4 consecutive channels, i.e. 8-byte runs of a row of Y; the
// epilogue passes each 32x32 tile through LDS so that a store instruction
// writes 64-byte row pieces.
//
// Pipeline: a workgroup owns a BM x BN output tile and walks K in stages of
// BK bytes (128 for the large tiles).  Stages go straight from global memory
// into LDS with buffer_load ... lds (no staging registers, no LDS store
// instructions).  The large tiles use a split ring: three slots for one
// operand and two for the other, so the first is requested two stages ahead
// and the second one (int8: W ahead, fp8: X ahead); the other tiles use a
// ring of S whole stages.  Chunks past K or rows past M/N are requested at
// an out-of-range buffer offset, which the hardware returns as zeros, so
// partial tiles need no branches and stages past the end add nothing.
// Fragments are read with 16-byte LDS reads, one MFMA K step ahead of the
// MFMAs that use them, including across the stage boundary.  16-byte chunks
// are XOR swizzled within each LDS row so that neither the DMA writes nor
// the fragment reads conflict on banks.  The accumulators stay in registers
// for the whole K loop; int32 never touches HBM on the fused path.
//
// Persistence: one workgroup per CU walks its share of the tiles.  On the
// 256x192 int8 tile the ring's requests past a tile's last stage fetch the
// next tile's first three stages during the last steps; the other split-ring
// tiles request the next tile's first stage before the epilogue.
//
// Workgroup order: consecutive workgroup ids are dispatched round robin over
// the 8 XCDs, each with its own L2.  Tiles are remapped so that each XCD gets
// a contiguous range, walked in groups of kGroupM tile rows, so the tiles
// resident on one XCD share X and W panels in its L2.
#include "kernels.h"
#include "epilogue.h"

#include <algorithm>
#include <type_traits>

namespace w8a8 {
namespace {

typedef int v4i __attribute__((ext_vector_type(4)));
typedef int v8i __attribute__((ext_vector_type(8)));
typedef int v16i __attribute__((ext_vector_type(16)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef float f32x2 __attribute__((ext_vector_type(2)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) void lds_void;

constexpr int kWave = 64;
constexpr int kNumXcd = 8;
constexpr int kGroupM = 4;
constexpr int kCUs = 256;               // compute units of an MI355X (one workgroup each)
constexpr int kDmaBytes = kWave * 16;    // one wavefront DMA: 64 lanes x 16 B
constexpr uint32_t kOOB = 0x80000000u;    // buffer offset beyond any tile: reads as zero
constexpr int kRsrcWord3 = 0x00020000;    // raw buffer, 32-bit data format (gfx9 family)
// Cache policy of the output stores: non-temporal (the NT bit of gfx94x/gfx950
// buffer instructions).  Y is written once and not read again by this kernel;
// streaming it keeps the operand panels in L2 and leaves fewer dirty lines for
// the kernel-end write-back (measured: DiT block GEMMs +2.6%, bit-identical).
constexpr int kStoreNT = 2;

// S >= 2: ring of S whole stages.  S == 0: split ring -- three slots of one
// operand and two of the other, so the first is requested two stages ahead
// and the second one (see the main loop).
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
  static constexpr int CPR = BK / 16;                // 16-byte chunks per LDS row
  static constexpr int kDmaRows = kDmaBytes / BK;    // rows moved by one wavefront DMA
  static constexpr int DX = BM / kDmaRows / kWaves;  // X DMAs per wavefront per stage
  static constexpr int DW = BN / kDmaRows / kWaves;  // W DMAs per wavefront per stage
  static constexpr int D = DX + DW;
  static constexpr int kStageBytes = (BM + BN) * BK;
  // Split ring: the operand requested two stages ahead ("A") has three
  // slots, lds0..2, the other ("B") two, lds3..4 (which operand is A is the
  // kernel's choice).  Otherwise lds0..S-1 hold whole stages.
  static constexpr int kSlots = kSplit ? 5 : S;
  static constexpr int kArrA_X = kSplit ? BM * BK : kStageBytes;   // slot sizes with A = X
  static constexpr int kArrB_X = kSplit ? BN * BK : kStageBytes;
  static constexpr int kLdsBytes = kSplit ? 3 * (BM > BN ? BM : BN) * BK + 2 * (BM > BN ? BN : BM) * BK
                                          : S * kStageBytes;
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
__device__ __forceinline__ void dma16(__amdgpu_buffer_rsrc_t r, int8_t* lds, uint32_t voffset,
                                      int soffset = 0) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_void*)lds, 16, (int)voffset, soffset, 0, 0);
}

__device__ __forceinline__ float bf16_to_float(uint16_t b) {
  return __uint_as_float((uint32_t)b << 16);
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

// Operand types.  int8: v_mfma_i32_32x32x32_i8, 16 K bytes per lane and
// step, int32 accumulators.  fp8 (e4m3): v_mfma_f32_32x32x64_f8f6f4 (the
// scaled form with unit E8M0 scales, 127), 32 K bytes per lane and step,
// fp32 accumulators.  Both take the lane's row of A and of B at the same K
// positions, so any fixed assignment of K bytes to (lane half, byte) that is
// the same for both operands gives the same dot products.
struct OpI8 {
  static constexpr bool kF8 = false;
  static constexpr int kStepK = 32;   // K bytes per MFMA
  typedef v4i Frag;
  typedef v16i Acc;
};
struct OpF8 {
  static constexpr bool kF8 = true;
  static constexpr int kStepK = 64;
  typedef v8i Frag;
  typedef v16f Acc;
};

// Output tile `t` (0 <= t < tiles_m * tiles_n) -> (first row, first channel).
// Tiles are spread so that each XCD works on a contiguous range, walked in
// groups of kGroupM tile rows (tiles resident on one XCD share X and W panels
// in its L2).  A workgroup on XCD x only ever gets tiles of XCD x's range:
// grid sizes are multiples of 8 whenever tile counts are.
__device__ __forceinline__ void tile_origin(int t, int tiles_m, int tiles_n, int bm, int bn,
                                            int& m0, int& n0) {
  const int ntiles = tiles_m * tiles_n;
  if (ntiles % kNumXcd == 0) {
    // XCD x walks its own range of tiles starting x rounds in (a round = the
    // 32 tiles its workgroups take at once), wrapping around: otherwise all
    // XCDs reach the same new weight columns in the same round and all wait
    // on HBM for them (the weights are cold at every use inside a model);
    // rotated, the columns an XCD reaches were read by another XCD a round
    // earlier and come from the Infinity Cache.  A cyclic shift within each
    // XCD's range keeps the mapping one to one; it is applied when the range
    // is whole rounds, so that every round stays one compact block of tiles.
    constexpr int kRound = kCUs / kNumXcd;
    const int x = t % kNumXcd, per_xcd = ntiles / kNumXcd;
    const int shift = per_xcd % kRound == 0 ? x * kRound : 0;
    t = x * per_xcd + (t / kNumXcd + shift) % per_xcd;
  }
  const int per_group = kGroupM * tiles_n;
  const int group = t / per_group;
  const int first_m = group * kGroupM;
  const int gsize = min(tiles_m - first_m, kGroupM);
  const int in_group = t - group * per_group;
  m0 = (first_m + in_group % gsize) * bm;
  n0 = (in_group / gsize) * bn;
}

// K split of a launch: the reduction of each output tile is cut into `chunks`
// equal ranges of K bytes, each its own work item, whose raw int32 sums go to
// their own output slice (`out_stride` elements apart); the kernel's K is then
// the length of one range and `ldk` the row length of X and W.  No split:
// chunks = 1, ldk = K.
struct KSplit {
  int ldk;
  int chunks;
  int64_t out_stride;
};

// Persistent kernel: gridDim.x workgroups (at most one per CU) walk the work
// items t = blockIdx.x, blockIdx.x + gridDim.x, ... (output tile t mod
// tiles, K range t / tiles).  With the split ring, the first two requests of
// a workgroup's next item are issued before the epilogue of the current one,
// so the epilogue hides their latency.
template <class T, Epilogue EPI, class Op>
__global__ __launch_bounds__(T::kThreads, 1) void gemm_i8_kernel(
    const int8_t* __restrict__ X, const int8_t* __restrict__ W, const float* __restrict__ sx,
    const float* __restrict__ sw, const uint16_t* __restrict__ bias, void* __restrict__ out,
    int M, int N, int K, int ldy, int tiles_m, int tiles_n, int vec_store, KSplit ks) {
  // Split ring, int8: A = W.  In a model the weights arrive cold from HBM at
  // every use while the activation codes were just written by the quantizer
  // (measured: +1.7% on the DiT block step, neutral with warm caches); the
  // fp8 tile keeps A = X, whose registers do not fit the other order.
  constexpr bool kWAhead = T::kSplit && !Op::kF8;
  constexpr int kArr012 = kWAhead ? T::kArrB_X : T::kArrA_X;
  constexpr int kArr34 = kWAhead ? T::kArrA_X : T::kArrB_X;
  // One array per ring slot: distinct objects let the compiler see that a
  // DMA into one slot never aliases fragment reads from another.
  __shared__ __attribute__((aligned(16))) int8_t lds0[kArr012];
  __shared__ __attribute__((aligned(16))) int8_t lds1[kArr012];
  __shared__ __attribute__((aligned(16))) int8_t lds2[T::kSlots > 2 ? kArr012 : 16];
  __shared__ __attribute__((aligned(16))) int8_t lds3[T::kSlots > 3 ? kArr34 : 16];
  __shared__ __attribute__((aligned(16))) int8_t lds4[T::kSlots > 4 ? kArr34 : 16];
  // Epilogue transpose regions and channel scales in an array of their own
  // where the split ring leaves room (256x192 int8): LDS writes to the ring's
  // slots would have to wait for the next tile's first requests in flight,
  // which the compiler cannot tell apart from them.
  constexpr int kEpiBytes = 8 * 32 * 64 + 2 * T::BN * 4;
  constexpr bool kEpiOwn = T::kSplit && 3 * kArr012 + 2 * kArr34 + kEpiBytes <= 160 * 1024;
  __shared__ __attribute__((aligned(16))) int8_t lds_epi[kEpiOwn ? kEpiBytes : 16];
  int8_t* const ring[4] = {lds0, lds1, lds2, lds3};

  const int ntiles = tiles_m * tiles_n;
  const int nitems = ntiles * ks.chunks;
  const int tid = threadIdx.x;
  const int lane = tid % kWave;
  const int wave = __builtin_amdgcn_readfirstlane(tid / kWave);
  const int wm = wave / T::WN, wn = wave % T::WN;
  const int row_in = lane % 32;   // row of the 32-row MFMA operand this lane feeds
  const int khalf = lane / 32;    // which 16-byte half of each 32-byte K step
  const int KT = (K + T::BK - 1) / T::BK;

  // ---- DMA addressing ----
  // Lane p of a DMA fills LDS slot p of a block of kDmaRows rows (DMA writes
  // are linear, hence conflict-free): row r = block*kDmaRows + p/CPR,
  // physical chunk p%CPR, so the lane fetches logical chunk swz(r, p%CPR).
  // Wavefront w moves blocks w, w + kWaves, ... of X and of W; the swizzle
  // repeats every 16 rows, so the chunk a lane fetches is the same in all of
  // them.  Its byte offset in stage 0 of a tile is the same for every tile:
  // rows past M (N) fall outside the tile's buffer resource, whose range
  // ends with the tile's last valid row, and read as zeros.
  //
  // With the 256x192 split ring only the first half of the wavefronts issue
  // stage requests (twice as many each); the other half only read fragments
  // and run MFMAs.  Measured on MI355X: the K loop runs about 4% faster than
  // with every wavefront issuing.  (The 256x256 tile has no registers for
  // the doubled request count, nor has the fp8 tile with the raw epilogue.)
  constexpr bool kHalfDma = T::kSplit && T::BN < 256 && EPI != Epilogue::kRawI32;
  constexpr int kDmaWaves = kHalfDma ? T::kWaves / 2 : T::kWaves;
  constexpr int DXk = T::BM / T::kDmaRows / kDmaWaves;   // X requests per DMA wavefront and stage
  constexpr int DWk = T::BN / T::kDmaRows / kDmaWaves;   // W requests
  static_assert(DXk * T::kDmaRows * kDmaWaves == T::BM && DWk * T::kDmaRows * kDmaWaves == T::BN,
                "DMA wavefronts move whole blocks of X and W");
  static_assert(2 * DXk + DWk <= 63 && 2 * DWk + DXk <= 63, "vmcnt range");
  static_assert((kDmaWaves * T::kDmaRows) % 16 == 0, "one swizzle phase per DMA block set");
  const bool dma_wave = !kHalfDma || wave < kDmaWaves;
  // Split ring with the bf16 epilogue: the epilogue's stores are buffer
  // stores, exactly two per 32x32 tile and wavefront, so the hand-over can
  // wait for the new tile's first requests without waiting for the stores
  // (the counter completes in order).  Offsets are 32-bit: the host sends
  // the plain path (vec_store = 0) when BM * ldy * 2 >= 2^31.
  constexpr bool kCountedStores = T::kSplit && EPI != Epilogue::kRawI32;
  constexpr int kStores = 2 * T::FM * T::FN;   // store instructions per wavefront and tile
  const int dma_r = (wave % kDmaWaves) * T::kDmaRows + lane / T::CPR;
  const int col = swz<T::CPR>(dma_r, lane % T::CPR) * 16;   // K byte offset within a stage
  const uint32_t off0 = (uint32_t)(dma_r * ks.ldk + col);
  const uint32_t blk_stride = (uint32_t)(kDmaWaves * T::kDmaRows * ks.ldk);

  // Per-item state (wavefront-uniform): origin, K range and buffer
  // resources over the tile's rows of X and W from the range's first byte;
  // each resource ends with the last valid row's last byte of the range
  // (rows past M or N read as zeros; bytes of a row past the range are never
  // requested: the K loop stops at the range's end).
  struct TileAddr {
    int m0, n0, c;
    __amdgpu_buffer_rsrc_t rx, rw;
  };
  auto setup = [&](int t, TileAddr& a) {
    a.c = t / ntiles;
    tile_origin(t - a.c * ntiles, tiles_m, tiles_n, T::BM, T::BN, a.m0, a.n0);
    const int rows_x = min(T::BM, M - a.m0), rows_w = min(T::BN, N - a.n0);
    const int64_t k0 = (int64_t)a.c * K;
    a.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(X + (int64_t)a.m0 * ks.ldk + k0), (short)0,
                                             (rows_x - 1) * ks.ldk + K, kRsrcWord3);
    a.rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(W + (int64_t)a.n0 * ks.ldk + k0), (short)0,
                                             (rows_w - 1) * ks.ldk + K, kRsrcWord3);
  };
  // Request the X (W) part of stage kt of tile `a` into `buf`; chunks at or
  // past K read as zeros.
  // `interior` (a std::bool_constant): the stage lies entirely inside K.
  // Then its K offset goes into the instruction's scalar offset, with no
  // per-lane arithmetic (the row, and with it the range check against the
  // tile's rows, stays in the vector offset); otherwise the out-of-range
  // offset is selected per lane for chunks past K.
  // The per-request offsets are formed at each request from an opaque copy
  // of off0 (one add, plus a select past K): hoisted out of the loops they
  // would hold 2 x DX + DW registers through the whole kernel.
  auto issue_rows = [&](__amdgpu_buffer_rsrc_t r, int n, int8_t* buf, int kt, auto interior) {
    const int kb = kt * T::BK;
    uint32_t o = off0;
    asm volatile("" : "+v"(o));
    if constexpr (decltype(interior)::value) {
#pragma unroll
      for (int i = 0; i < n; ++i)
        dma16(r, buf + (wave + i * kDmaWaves) * kDmaBytes, o + (uint32_t)(i * blk_stride), kb);
    } else {
      const bool in_k = kb + col < K;
#pragma unroll
      for (int i = 0; i < n; ++i)
        dma16(r, buf + (wave + i * kDmaWaves) * kDmaBytes,
              in_k ? o + (uint32_t)(i * blk_stride + kb) : kOOB);
    }
  };
  auto issue_x = [&](const TileAddr& a, int8_t* buf, int kt, auto interior) {
    issue_rows(a.rx, DXk, buf, kt, interior);
  };
  auto issue_w = [&](const TileAddr& a, int8_t* buf, int kt, auto interior) {
    issue_rows(a.rw, DWk, buf, kt, interior);
  };
  // split ring: A = the operand with three slots, B = the one with two
  auto issue_a = [&](const TileAddr& a, int8_t* buf, int kt, auto interior) {
    if constexpr (kWAhead) issue_w(a, buf, kt, interior);
    else issue_x(a, buf, kt, interior);
  };
  auto issue_b = [&](const TileAddr& a, int8_t* buf, int kt, auto interior) {
    if constexpr (kWAhead) issue_x(a, buf, kt, interior);
    else issue_w(a, buf, kt, interior);
  };
  // With the epilogue in an LDS array of its own, the ring's requests for
  // stages past the tile's last one (KT6 .. KT6 + 2) are the next tile's
  // stages 0 .. 2, into exactly the slots its first steps read: the next
  // tile's start is requested during this tile's last steps, and the tile
  // boundary needs no requests, waits or barriers of its own.
  TileAddr pre;        // the next tile (rows out of range when there is none)
  int kt6_cur = 0;     // stages of the current tile's ring walk
  auto issue_a_at = [&](const TileAddr& a, int8_t* buf, int s, auto interior) {
    if (s >= kt6_cur) issue_a(pre, buf, s - kt6_cur, std::false_type{});
    else issue_a(a, buf, s, interior);
  };
  auto issue_b_at = [&](const TileAddr& a, int8_t* buf, int s, auto interior) {
    if (s >= kt6_cur) issue_b(pre, buf, s - kt6_cur, std::false_type{});
    else issue_b(a, buf, s, interior);
  };
  constexpr int DA = kWAhead ? DWk : DXk;   // requests per stage of A, B
  constexpr int DB = kWAhead ? DXk : DWk;
  static_assert(2 * DA + DB + kStores <= 63, "vmcnt range");
  // Whole stage kt into ring slot `buf` (X rows first, then W rows).
  auto issue = [&](const TileAddr& a, int8_t* buf, int kt, auto interior) {
    issue_x(a, buf, kt, interior);
    issue_w(a, buf + T::BM * T::BK, kt, interior);
  };
  // The 256x256 tile keeps one (checked) loop: it has no registers to spare
  // for a second copy of the DMA offsets.
  constexpr bool kSplitK = T::BM * T::BN < 256 * 256;
  const std::false_type kChecked;
  const std::true_type kInterior;
  const std::true_type kDmaRole;    // K loop of a wavefront that issues the stage requests
  const std::false_type kMmaRole;   // ... of one that does not

  constexpr int KSUB = T::BK / Op::kStepK;   // MFMA K steps per stage
  constexpr int CPS = Op::kStepK / 32;        // 16-byte chunks per lane and K step
  static_assert(KSUB >= 1, "a stage holds at least one MFMA K step");
  typename Op::Acc acc[T::FM][T::FN];

  // Fragment registers, double buffered by MFMA K step parity (int8); the
  // fp8 fragments are twice as wide and single buffered, which keeps the
  // 128 accumulators and both operands within 256 VGPRs.  In K step s lane
  // half h reads chunks (2s + h)*CPS ... + CPS-1 of its row.
  constexpr int NB = Op::kF8 ? 1 : 2;
  typename Op::Frag fa[NB][T::FN], fb[NB][T::FM];
  auto read_frag = [&](const int8_t* base, int r, int c) {
    typename Op::Frag f;
    if constexpr (CPS == 1) {
      f = *reinterpret_cast<const v4i*>(base + r * T::BK + swz<T::CPR>(r, c) * 16);
    } else {
      const v4i lo = *reinterpret_cast<const v4i*>(base + r * T::BK + swz<T::CPR>(r, c) * 16);
      const v4i hi = *reinterpret_cast<const v4i*>(base + r * T::BK + swz<T::CPR>(r, c + 1) * 16);
      f = v8i{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
    }
    return f;
  };
  auto frag2 = [&](const int8_t* xs, const int8_t* ws, int s, int slot) {
    slot %= NB;
    const int c = (s * 2 + khalf) * CPS;
#pragma unroll
    for (int j = 0; j < T::FN; ++j) fa[slot][j] = read_frag(ws, wn * T::TN + j * 32 + row_in, c);
#pragma unroll
    for (int i = 0; i < T::FM; ++i) fb[slot][i] = read_frag(xs, wm * T::TM + i * 32 + row_in, c);
  };
  auto frag = [&](const int8_t* buf, int s, int slot) { frag2(buf, buf + T::BM * T::BK, s, slot); };
  // fragments from an A slot and a B slot of the split ring
  auto frag_ab = [&](const int8_t* as, const int8_t* bs, int s, int slot) {
    if constexpr (kWAhead) frag2(bs, as, s, slot);
    else frag2(as, bs, s, slot);
  };
  auto mfmas = [&](int slot) {
    slot %= NB;
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) {
        if constexpr (Op::kF8)
          acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
              fa[slot][j], fb[slot][i], acc[i][j], 0, 0, 0, 127, 0, 127);
        else
          acc[i][j] = __builtin_amdgcn_mfma_i32_32x32x32_i8(fa[slot][j], fb[slot][i], acc[i][j], 0, 0, 0);
      }
  };

  // Scheduling of the code after a barrier: the next stage's first fragment
  // reads, then the last K step's MFMAs each followed by one stage request
  // (and its address arithmetic), so the MFMA pipe restarts right away.
  // A requesting wavefront places ceil(requests / MFMAs) stage requests
  // after each MFMA; one that makes no requests only orders its fragment
  // reads before its MFMAs.
  auto interleave = [&](auto role) {
    __builtin_amdgcn_sched_group_barrier(0x100, (T::FM + T::FN) * CPS, 0);   // fragment reads
    if constexpr (decltype(role)::value) {
      constexpr int kPer = (DXk + DWk + T::FM * T::FN - 1) / (T::FM * T::FN);
#pragma unroll
      for (int q = 0; q < T::FM * T::FN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3 * kPer, 0);      // address VALU
        __builtin_amdgcn_sched_group_barrier(0x020, kPer, 0);          // DMAs
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, T::FM * T::FN, 0);   // the MFMAs
    }
    __builtin_amdgcn_sched_barrier(0);
  };
  // Single-buffered fragments: the MFMAs of a K step go before the reads of
  // the next step's fragments into the same registers.
  auto interleave1 = [&](auto role) {
    if constexpr (decltype(role)::value) {
      constexpr int kPer = (DXk + DWk + T::FM * T::FN - 1) / (T::FM * T::FN);
#pragma unroll
      for (int q = 0; q < T::FM * T::FN; ++q) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);             // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, 3 * kPer, 0);      // address VALU
        __builtin_amdgcn_sched_group_barrier(0x020, kPer, 0);          // DMAs
      }
    } else {
      __builtin_amdgcn_sched_group_barrier(0x008, T::FM * T::FN, 0);   // the MFMAs
    }
    __builtin_amdgcn_sched_group_barrier(0x100, (T::FM + T::FN) * CPS, 0);   // fragment reads
    __builtin_amdgcn_sched_barrier(0);
  };

  // Step k (stage k in slot `cur`, fragments of its first K step in flight):
  // run the K steps; once every wavefront is past its reads of `cur` and
  // stage k+1 has landed (one barrier), request stage k+S into `cur` and
  // start reading stage k+1's first fragments under the MFMAs of the last K
  // step.  A stage is thus requested a full S-1 steps before it is needed.
  auto step = [&](const TileAddr& a, int8_t* cur, int8_t* nxt, int k, auto interior) {
    if constexpr (NB == 1) {
#pragma unroll
      for (int s = 0; s + 1 < KSUB; ++s) {
        mfmas(0);
        __builtin_amdgcn_sched_barrier(0);
        frag(cur, s + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_lgkmcnt0();
      wait_vmcnt<(T::S - 2) * T::D>();
      barrier();
      issue(a, cur, k + T::S, interior);
      mfmas(0);
      frag(nxt, 0, 0);
      interleave1(kDmaRole);
      return;
    }
#pragma unroll
    for (int s = 0; s + 1 < KSUB; ++s) {
      frag(cur, s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkmcnt0();                 // this wavefront's reads of `cur` are done
    wait_vmcnt<(T::S - 2) * T::D>();  // its DMAs of stage k+1 have landed
    barrier();                       // ... and everyone's
    frag(nxt, 0, KSUB & 1);
    issue(a, cur, k + T::S, interior);
    mfmas((KSUB - 1) & 1);
    interleave(kDmaRole);
  };

  // Dequant scalars of the current tile: per-token scales of the rows this
  // lane holds, and (threads below BN) one channel's scale and bias (kept
  // as bf16 bits until the epilogue).  With the epilogue's own LDS they are
  // requested at the first step of the tile's last six, after that step's
  // wait and before its requests, so the next explicit wait covers them;
  // otherwise at the tile's start (its K loop ends with a full wait).
  // Requested and used within one tile,
  // they are never live across the tile loop's back edge, where a pending
  // load in a loop-carried register would make the compiler wait for every
  // outstanding request (next-tile stages and output stores included).
  float sa_n[T::FM], sw_n = 0.0f;
  uint32_t b_n = 0;
  auto load_scalars = [&](const TileAddr& a) {
    if constexpr (EPI != Epilogue::kRawI32) {
#pragma unroll
      for (int i = 0; i < T::FM; ++i) sa_n[i] = sx[min(a.m0 + wm * T::TM + i * 32 + row_in, M - 1)];
      static_assert(T::BN <= T::kThreads, "one thread per channel of the block");
      sw_n = 0.0f;
      b_n = 0;
      if (tid < T::BN && a.n0 + tid < N) {
        sw_n = sw[a.n0 + tid];
        if (bias != nullptr) b_n = bias[a.n0 + tid];
      }
    }
  };

  // Split-ring step k: A_k in `ac`, B_k in `bc`, stage k+1 in `an`/`bn1`.
  // After the barrier that frees A_k's and B_k's slots, B_{k+2} and then
  // A_{k+3} are requested into them: at the next barrier only the B part
  // (requested one step earlier) is on the critical path, while A has two
  // steps to land.  With `pend_out` the A request is left to the next step,
  // which makes it (`pend_in`, into slot `ap`) alongside its first K step's
  // MFMAs; it is still that step's last request before its wait, so the
  // wait's count is unchanged.
  auto step_split = [&](const TileAddr& a, int8_t* ac, int8_t* bc, int8_t* an, int8_t* bn1,
                        int k, auto interior, auto role, auto fin, auto loads, auto pend_in, auto pend_out,
                        int8_t* ap) __attribute__((always_inline)) {
    constexpr bool kDma = decltype(role)::value;
    constexpr bool kFin = decltype(fin)::value;   // last six steps: requests may reach the next tile
    if constexpr (NB == 1) {
#pragma unroll
      for (int s = 0; s + 1 < KSUB; ++s) {
        mfmas(0);
        __builtin_amdgcn_sched_barrier(0);
        frag_ab(ac, bc, s + 1, 0);
        __builtin_amdgcn_sched_barrier(0);
      }
      wait_lgkmcnt0();
      if constexpr (kDma) wait_vmcnt<DA>();
      barrier();
      if constexpr (decltype(loads)::value) load_scalars(a);
      if constexpr (kDma && kFin) {
        issue_b_at(a, bc, k + 2, interior);
        issue_a_at(a, ac, k + 3, interior);
      } else if constexpr (kDma) {
        issue_b(a, bc, k + 2, interior);
        issue_a(a, ac, k + 3, interior);
      }
      mfmas(0);
      frag_ab(an, bn1, 0, 0);
      interleave1(role);
      return;
    }
    {
      frag_ab(ac, bc, 1, 1);
      if constexpr (kDma && decltype(pend_in)::value) {
        // the previous step's A request, spread over this step's first MFMAs
        if constexpr (kFin) issue_a_at(a, ap, k + 2, interior);
        else issue_a(a, ap, k + 2, interior);
      }
      mfmas(0);
      if constexpr (kDma && decltype(pend_in)::value) {
        __builtin_amdgcn_sched_group_barrier(0x100, (T::FM + T::FN) * CPS, 0);
#pragma unroll
        for (int q = 0; q < T::FM * T::FN; ++q) {
          __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
          __builtin_amdgcn_sched_group_barrier(0x002, 3, 0);
          __builtin_amdgcn_sched_group_barrier(0x020, 1, 0);
        }
      }
      __builtin_amdgcn_sched_barrier(0);
    }
#pragma unroll
    for (int s = 1; s + 1 < KSUB; ++s) {
      frag_ab(ac, bc, s + 1, (s + 1) & 1);
      __builtin_amdgcn_sched_barrier(0);
      mfmas(s & 1);
      __builtin_amdgcn_sched_barrier(0);
    }
    wait_lgkmcnt0();
    if constexpr (kDma) wait_vmcnt<DA>();   // everything but A_{k+2} (the last request) has landed
    barrier();
    frag_ab(an, bn1, 0, KSUB & 1);
    if constexpr (decltype(loads)::value) load_scalars(a);
    if constexpr (kDma && kFin) {
      issue_b_at(a, bc, k + 2, interior);
      if constexpr (!decltype(pend_out)::value) issue_a_at(a, ac, k + 3, interior);
    } else if constexpr (kDma) {
      issue_b(a, bc, k + 2, interior);
      if constexpr (!decltype(pend_out)::value) issue_a(a, ac, k + 3, interior);
    }
    mfmas((KSUB - 1) & 1);
    interleave(role);
  };

  // ---- epilogue placement in LDS (the ring is free after a tile's K loop) ----
  // Split ring: the transpose regions start at lds1 and the scales/bias come
  // after them, leaving lds0 and lds3 to the next tile's first requests.
  // Otherwise the regions start at lds0.
  constexpr int kRegion = 32 * 64;   // per wavefront: 32 rows x 32 bf16 channels
  constexpr bool kSbAfter = T::kWaves * kRegion + 2 * T::BN * 4 <= kArr012;
  static_assert(T::kWaves * kRegion <= kArr012, "regions fit in one array");
  static_assert(kSbAfter || (!T::kSplit && 2 * T::BN * 4 <= kArr012), "scales and bias fit");
  static_assert(!kEpiOwn || T::kWaves == 8, "regions of eight wavefronts");
  int8_t* const reg_a = kEpiOwn ? lds_epi : T::kSplit ? lds1 : lds0;
  // channel scales and biases (fp32) follow the regions, else take the next array
  int8_t* const sb_arr = kEpiOwn || kSbAfter ? reg_a + T::kWaves * kRegion : lds1;


  TileAddr cur;
  setup(blockIdx.x, cur);
  if constexpr (T::kSplit) {
    // A slots lds0..lds2 (A_k in slot k%3), B slots lds3, lds4 (B_k in k%2);
    // the slot pattern repeats every 6 stages.
    if (dma_wave) {
      issue_a(cur, lds0, 0, kChecked);
      issue_b(cur, lds3, 0, kChecked);
      issue_a(cur, lds1, 1, kChecked);
      issue_b(cur, lds4, 1, kChecked);
      issue_a(cur, lds2, 2, kChecked);
      wait_vmcnt<2 * DA + DB>();
    }
    barrier();
    frag_ab(lds0, lds3, 0, 0);
  }

  for (int t = blockIdx.x; t < nitems; t += gridDim.x) {
#pragma unroll
    for (int i = 0; i < T::FM; ++i)
#pragma unroll
      for (int j = 0; j < T::FN; ++j) acc[i][j] = typename Op::Acc{};

    // ---- K loop ----
    if constexpr (!kEpiOwn) load_scalars(cur);
    if constexpr (T::kSplit) {
      const int KT6 = (KT + 5) / 6 * 6;   // padding stages read as zeros
      // six steps of the ring; the requests they make reach stage kt + 8
      auto kloop = [&](auto role) __attribute__((always_inline)) {
        // `last`: the tile's last six steps, whose first one requests the
        // dequant scalars
        auto six = [&](int kt, auto interior, auto fin, auto last) __attribute__((always_inline)) {
          // int8: steps 0-4 of the six leave their A request to the next
          // step's first K step (`ap` is the slot it goes to), so a step's
          // requests do not all queue behind one barrier
          constexpr std::false_type no{};
          constexpr std::integral_constant<bool, !Op::kF8> d{};
          step_split(cur, lds0, lds3, lds1, lds4, kt, interior, role, fin, last, no, d, lds2);
          step_split(cur, lds1, lds4, lds2, lds3, kt + 1, interior, role, fin, no, d, d, lds0);
          step_split(cur, lds2, lds3, lds0, lds4, kt + 2, interior, role, fin, no, d, d, lds1);
          step_split(cur, lds0, lds4, lds1, lds3, kt + 3, interior, role, fin, no, d, d, lds2);
          step_split(cur, lds1, lds3, lds2, lds4, kt + 4, interior, role, fin, no, d, d, lds0);
          step_split(cur, lds2, lds4, lds0, lds3, kt + 5, interior, role, fin, no, d, no, lds1);
        };
        constexpr std::true_type last{};
        constexpr std::false_type not_last{};
        int kt = 0;
        if constexpr (kSplitK)
          for (; kt < KT6 && (kt + 9) * T::BK <= K; kt += 6) six(kt, kInterior, std::false_type{}, not_last);
        if constexpr (kEpiOwn) {
          for (; kt < KT6 - 6; kt += 6) six(kt, kChecked, std::false_type{}, not_last);
          if constexpr (decltype(role)::value) {
            kt6_cur = KT6;
            if (t + (int)gridDim.x < nitems) {
              setup(t + (int)gridDim.x, pre);
            } else {
              pre.m0 = pre.n0 = 0;
              pre.rx = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(X), (short)0, 0, kRsrcWord3);
              pre.rw = __builtin_amdgcn_make_buffer_rsrc(const_cast<int8_t*>(W), (short)0, 0, kRsrcWord3);
            }
          }
          six(kt, kChecked, std::true_type{}, last);
          // wavefronts without requests of their own: their scalar loads
          // (six steps old) are the only ones that may be outstanding
          if constexpr (!decltype(role)::value) wait_vmcnt<0>();
        } else {
          for (; kt < KT6; kt += 6) six(kt, kChecked, std::false_type{}, not_last);
        }
      };
      if constexpr (kHalfDma) {
        if (dma_wave) kloop(kDmaRole);
        else kloop(kMmaRole);
      } else {
        kloop(kDmaRole);
      }
    } else {
#pragma unroll
      for (int s = 0; s < T::S; ++s) issue(cur, ring[s], s, kChecked);
      wait_vmcnt<(T::S - 1) * T::D>();
      barrier();
      frag(ring[0], 0, 0);
      const int KTr = (KT + T::S - 1) / T::S * T::S;   // padding stages read as zeros
      // S steps of the ring; the requests they make reach stage kt + 2S - 1
      auto round = [&](int kt, auto interior) {
        if constexpr (T::S == 2) {
          step(cur, lds0, lds1, kt, interior);
          step(cur, lds1, lds0, kt + 1, interior);
        } else if constexpr (T::S == 3) {
          step(cur, lds0, lds1, kt, interior);
          step(cur, lds1, lds2, kt + 1, interior);
          step(cur, lds2, lds0, kt + 2, interior);
        } else {
          step(cur, lds0, lds1, kt, interior);
          step(cur, lds1, lds2, kt + 1, interior);
          step(cur, lds2, lds3, kt + 2, interior);
          step(cur, lds3, lds0, kt + 3, interior);
        }
      };
      int kt = 0;
      if constexpr (kSplitK)
        for (; kt < KTr && (kt + 2 * T::S) * T::BK <= K; kt += T::S) round(kt, kInterior);
      for (; kt < KTr; kt += T::S) round(kt, kChecked);
    }
    if constexpr (!kEpiOwn) {
      wait_vmcnt<0>();
      wait_lgkmcnt0();
      barrier();   // every DMA and fragment read of this tile is done
    }

    const int m0 = cur.m0, n0 = cur.n0;
    [[maybe_unused]] const int c0 = cur.c;
    // output rows of this tile as a buffer range (bf16, ldy apart)
    __amdgpu_buffer_rsrc_t y_rsrc;
    if constexpr (kCountedStores)
      y_rsrc = __builtin_amdgcn_make_buffer_rsrc(
          reinterpret_cast<uint16_t*>(out) + (int64_t)m0 * ldy, (short)0,
          (int)((uint32_t)min(T::BM, M - m0) * (uint32_t)ldy * 2u), kRsrcWord3);
    const int t_next = t + gridDim.x;
    const bool has_next = t_next < nitems;

    // ---- epilogue: lane holds token m, channels n = base + 8*g + 4*khalf + 0..3 ----
    if constexpr (EPI != Epilogue::kRawI32) {
      // Lane-derived epilogue addresses are recomputed per tile (the opaque
      // copy of the lane id keeps them from being hoisted out of the tile
      // loop, where they would occupy registers through the K loop).
      int e_lane = lane;
      asm volatile("" : "+v"(e_lane));
      const int e_row = e_lane % 32, e_kh = e_lane / 32;
      // byte offset of this lane's 8 channels in its output row of a store
      const uint32_t y_lane = ((uint32_t)(e_lane / 4) * (uint32_t)ldy + (uint32_t)(e_lane % 4) * 8u) * 2u;
      float sa[T::FM];
#pragma unroll
      for (int i = 0; i < T::FM; ++i) sa[i] = sa_n[i];
      const float sw_l = sw_n, b_l = bf16_to_float((uint16_t)b_n);
      TileAddr nxt;
      if (has_next) setup(t_next, nxt);
      if constexpr (T::kSplit && !kEpiOwn) {
        if (has_next && dma_wave) {
          issue_a(nxt, lds0, 0, kChecked);
          issue_b(nxt, lds3, 0, kChecked);
        }
      }
      // The block's channel scales and bias (as fp32) go to LDS once, so each
      // group of 4 outputs needs two 16-byte LDS reads instead of 8 global loads.
      float* s_lds = reinterpret_cast<float*>(sb_arr);
      float* b_lds = s_lds + T::BN;
      if (tid < T::BN) {
        s_lds[tid] = sw_l;
        b_lds[tid] = b_l;
      }
      // LDS writes done, then a plain barrier: a full __syncthreads() fence
      // would also wait for the next tile's requests in flight
      wait_lgkmcnt0();
      barrier();
      // Column tiles j (32 channels) one at a time: the scales and biases of
      // this lane's 16 channels of j are read from LDS once for all FM row
      // tiles, and each 32x32 output tile is turned around in the
      // wavefront's own 2 KB LDS region (32 rows of 64 bytes) so that a
      // store instruction writes 16 whole 64-byte row pieces instead of 64
      // scattered 8-byte ones.
      int8_t* const region = reg_a + wave * kRegion;
      // 16-byte chunk c of region row r sits at chunk c ^ ((r/4) % 4), and in
      // rows 16..31 its two 8-byte halves are swapped: the writes (8 bytes
      // for each of 32 rows per half-wavefront) then cover all 64 banks once,
      // and the reads (16 bytes for 4 rows x 4 chunks per quarter-wavefront)
      // fill one 256-byte window.
      auto rsw = [](int r, int c) { return c ^ ((r >> 2) & 3); };
      f32x4 sv[4], bv[4];
      // this lane's channel scales and biases of column tile j
      auto load_sb = [&](int j) {
        const int nj = wn * T::TN + j * 32;
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          sv[g] = *reinterpret_cast<const f32x4*>(s_lds + nj + g * 8 + e_kh * 4);
          bv[g] = *reinterpret_cast<const f32x4*>(b_lds + nj + g * 8 + e_kh * 4);
        }
      };
      // 4 bf16 outputs (two packed words) of each run g of output tile (i, j):
      // channels nj + 8g + 4*khalf + 0..3
      uint32_t w[4][2];
      auto pack = [&](int i, int j) {
        const typename Op::Acc& c = acc[i][j];
        // the fp32 output value (GELU applied for the gelu epilogue)
        auto val = [&](int e, float s_w, float b) {
          const float y = dequant((float)c[e], sa[i], s_w, b);
          if constexpr (EPI == Epilogue::kBf16GeluScaleBias) return gelu(y);
          else return y;
        };
#pragma unroll
        for (int g = 0; g < 4; ++g) {
          const bf16x2 lo = __builtin_convertvector(
              (f32x2{val(g * 4, sv[g][0], bv[g][0]), val(g * 4 + 1, sv[g][1], bv[g][1])}), bf16x2);
          const bf16x2 hi = __builtin_convertvector(
              (f32x2{val(g * 4 + 2, sv[g][2], bv[g][2]), val(g * 4 + 3, sv[g][3], bv[g][3])}), bf16x2);
          w[g][0] = __builtin_bit_cast(uint32_t, lo);
          w[g][1] = __builtin_bit_cast(uint32_t, hi);
        }
      };
      if (vec_store) {
        // Software pipeline over the FM x FN output tiles b (column tile j =
        // b / FM, row tile i = b % FM): tile b's turn-around reads are in
        // flight while tile b+1 is converted, and tile b+1 is written to the
        // region once tile b's reads have returned (they feed its stores).
        constexpr int NB = T::FM * T::FN;
        auto put = [&]() {
#pragma unroll
          for (int g = 0; g < 4; ++g)
            *reinterpret_cast<u32x2*>(region + e_row * 64 + rsw(e_row, g) * 16 +
                                      8 * (e_kh ^ (e_row >> 4))) = u32x2{w[g][0], w[g][1]};
        };
        // The scales and biases of a new column tile are read as soon as the
        // previous one's last output tile is converted, a whole output tile
        // ahead of their use -- where the registers allow (up to 6 output
        // tiles per wavefront; with more, the early copy spills).
        constexpr bool kSbAhead = NB <= 6;
        auto pack_next = [&](int x) {
          if constexpr (!kSbAhead)
            if (x > 0 && x % T::FM == 0) load_sb(x / T::FM);
          pack(x % T::FM, x / T::FM);
          if constexpr (kSbAhead)
            if (x + 1 < NB && (x + 1) % T::FM == 0) load_sb((x + 1) / T::FM);
        };
        load_sb(0);
        pack_next(0);
        put();
#pragma unroll
        for (int b = 0; b < NB; ++b) {
          const int j = b / T::FM, i = b % T::FM;
          v4i v[2];
#pragma unroll
          for (int it = 0; it < 2; ++it) {
            const int r = it * 16 + e_lane / 4;
            v[it] = *reinterpret_cast<const v4i*>(region + r * 64 + rsw(r, e_lane % 4) * 16);
          }
          if (b + 1 < NB) pack_next(b + 1);
          v[1] = v4i{v[1][2], v[1][3], v[1][0], v[1][1]};   // rows 16..31: halves swapped
          const int nj = wn * T::TN + j * 32;
          const int mb = m0 + wm * T::TM + i * 32;   // first token of row tile i
          const int n = n0 + nj + (e_lane % 4) * 8;   // this lane's 8 channels when storing
          if constexpr (kCountedStores) {
            // exactly two store instructions per 32x32 tile: rows past M
            // fall outside the tile's buffer range, channels past N go to
            // the out-of-range offset
#pragma unroll
            for (int it = 0; it < 2; ++it) {
              const uint32_t o_tile = ((uint32_t)(mb - m0 + it * 16) * (uint32_t)ldy + (uint32_t)(n0 + nj)) * 2u;
              uint32_t o = n < N ? y_lane + o_tile : kOOB;
              asm volatile("" : "+v"(o));   // one store for all lanes, not one per branch
              __builtin_amdgcn_raw_buffer_store_b128(v[it], y_rsrc, o, 0, kStoreNT);
            }
          } else {
#pragma unroll
            for (int it = 0; it < 2; ++it) {
              const int m = mb + it * 16 + e_lane / 4;
              if (m < M && n < N)
                *reinterpret_cast<v4i*>(reinterpret_cast<uint16_t*>(out) + (int64_t)m * ldy + n) = v[it];
            }
          }
          if (b + 1 < NB) put();
        }
      } else {
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
          const int nj = wn * T::TN + j * 32;
          load_sb(j);
#pragma unroll
          for (int i = 0; i < T::FM; ++i) {
            pack(i, j);
            const int m = m0 + wm * T::TM + i * 32 + e_row;
            if (m < M) {
              uint16_t* yrow = reinterpret_cast<uint16_t*>(out) + (int64_t)m * ldy;
#pragma unroll
              for (int g = 0; g < 4; ++g) {
                const int n = n0 + nj + g * 8 + e_kh * 4;
                const uint16_t h[4] = {(uint16_t)w[g][0], (uint16_t)(w[g][0] >> 16), (uint16_t)w[g][1],
                                       (uint16_t)(w[g][1] >> 16)};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                  if (n + e < N) yrow[n + e] = h[e];
              }
            }
          }
        }
      }
      if (has_next) cur = nxt;
    } else {
      TileAddr nxt;
      if (has_next) setup(t_next, nxt);
      if constexpr (T::kSplit && !kEpiOwn) {
        if (has_next && dma_wave) {
          issue_a(nxt, lds0, 0, kChecked);
          issue_b(nxt, lds3, 0, kChecked);
        }
      }
#pragma unroll
      for (int i = 0; i < T::FM; ++i) {
        const int m = m0 + wm * T::TM + i * 32 + row_in;
        if (m >= M) continue;
        int32_t* crow = reinterpret_cast<int32_t*>(out) + (int64_t)c0 * ks.out_stride + (int64_t)m * ldy;
#pragma unroll
        for (int j = 0; j < T::FN; ++j) {
#pragma unroll
          for (int g = 0; g < 4; ++g) {
            const int n = n0 + wn * T::TN + j * 32 + g * 8 + khalf * 4;
            // raw accumulators (fp8: the fp32 bits).  The whole vector is
            // reinterpreted: bit-casting single fp32 elements of the fp8 MFMA's
            // result miscompiles (every element is taken to equal element 0).
            const v16i av = __builtin_bit_cast(v16i, acc[i][j]);
            int32_t a4[4];
#pragma unroll
            for (int e = 0; e < 4; ++e) a4[e] = av[g * 4 + e];
            if (vec_store && n + 3 < N) {
              *reinterpret_cast<v4i*>(crow + n) = v4i{a4[0], a4[1], a4[2], a4[3]};
            } else {
#pragma unroll
              for (int e = 0; e < 4; ++e)
                if (n + e < N) crow[n + e] = a4[e];
            }
          }
        }
      }
      if (has_next) cur = nxt;
    }

    // ---- hand over to the next tile ----
    if constexpr (kEpiOwn) {
      // the next tile's stages 0..2 were requested during the last steps of
      // this one, and stage 0 had landed by the last step's barrier
      if (has_next) frag_ab(lds0, lds3, 0, 0);
    } else if (has_next) {
      wait_lgkmcnt0();
      barrier();   // the epilogue's LDS regions and scales are free again
      if constexpr (T::kSplit) {
        if (dma_wave) {
          issue_a(cur, lds1, 1, kChecked);
          issue_b(cur, lds4, 1, kChecked);
          issue_a(cur, lds2, 2, kChecked);
          // A_0, B_0 of the new tile have landed (with counted stores these
          // drain under the new tile's first stage; otherwise they are
          // older than A_0, B_0 for the counter and are waited for too)
          if (kCountedStores && vec_store) wait_vmcnt<2 * DA + DB + kStores>();
          else wait_vmcnt<2 * DA + DB>();
        }
        barrier();
        frag_ab(lds0, lds3, 0, 0);
      }
    }
  }
  // requests of a last tile's final steps (the next tile's stages, out of
  // range) may still be writing LDS: drain them before the workgroup ends
  wait_vmcnt<0>();
}

// Compute units of the current device (each persistent workgroup takes one).
int num_cus() {
  int dev = 0, n = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0)
    return 256;
  return n / kNumXcd * kNumXcd > 0 ? n / kNumXcd * kNumXcd : n;
}

// Launch tile configuration T on the sub-problem M x N x K whose output rows
// are `ldy` elements apart (K the length of one K range when `ks` splits it).
template <class T, class Op>
hipError_t launch_t(Epilogue epi, const int8_t* xq, const int8_t* wq, const float* sx,
                    const float* sw, const uint16_t* bias, void* out, int64_t M, int64_t N,
                    int64_t K, int64_t ldy, hipStream_t stream, KSplit ks) {
  const int tiles_m = (int)((M + T::BM - 1) / T::BM);
  const int tiles_n = (int)((N + T::BN - 1) / T::BN);
  // at most one workgroup per CU (the tiles occupy a whole CU); a multiple
  // of the 8 XCDs so that each workgroup stays on its XCD's tile range
  const dim3 grid((unsigned)std::min<int64_t>((int64_t)tiles_m * tiles_n * ks.chunks, num_cus()));
  const dim3 block(T::kThreads);
  const uintptr_t o = reinterpret_cast<uintptr_t>(out);
  if (epi == Epilogue::kBf16ScaleBias) {
    // 16-byte stores; the split ring's buffer stores take 32-bit offsets
    // within a tile's rows
    const int vec = (ldy % 8 == 0) && (o % 16 == 0) && (int64_t)T::BM * ldy * 2 < (int64_t(1) << 31);
    hipLaunchKernelGGL((gemm_i8_kernel<T, Epilogue::kBf16ScaleBias, Op>), grid, block, 0, stream, xq,
                       wq, sx, sw, bias, out, (int)M, (int)N, (int)K, (int)ldy, tiles_m, tiles_n,
                       vec, ks);
  } else if (epi == Epilogue::kBf16GeluScaleBias) {
    // 16-byte stores; the split ring's buffer stores take 32-bit offsets
    // within a tile's rows
    const int vec = (ldy % 8 == 0) && (o % 16 == 0) && (int64_t)T::BM * ldy * 2 < (int64_t(1) << 31);
    hipLaunchKernelGGL((gemm_i8_kernel<T, Epilogue::kBf16GeluScaleBias, Op>), grid, block, 0, stream,
                       xq, wq, sx, sw, bias, out, (int)M, (int)N, (int)K, (int)ldy, tiles_m,
                       tiles_n, vec, ks);
  } else {
    const int vec = (ldy % 4 == 0) && (o % 16 == 0);
    hipLaunchKernelGGL((gemm_i8_kernel<T, Epilogue::kRawI32, Op>), grid, block, 0, stream, xq, wq,
                       nullptr, nullptr, nullptr, out, (int)M, (int)N, (int)K, (int)ldy, tiles_m,
                       tiles_n, vec, ks);
  }
  return hipGetLastError();
}

// Compiled tile configurations.
using CfgSplit = Tile<256, 256, 128, 2, 4, 0>;   // 256x256, split ring
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

template <class Op>
hipError_t launch_cfg(int cfg, Epilogue epi, const int8_t* xq, const int8_t* wq, const float* sx,
                      const float* sw, const uint16_t* bias, void* out, int64_t M, int64_t N,
                      int64_t K, int64_t ldy, hipStream_t s, KSplit ks) {
  switch (cfg) {
    case kSplit256: return launch_t<CfgSplit, Op>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s, ks);
    case kWhole256: return launch_t<CfgWhole, Op>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s, ks);
    case k192: return launch_t<Cfg192, Op>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s, ks);
    case kTail128x256: return launch_t<CfgTail, Op>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s, ks);
    case k256x128: return launch_t<Cfg256x128, Op>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s, ks);
    case k128: return launch_t<Cfg128, Op>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s, ks);
    case k64: return launch_t<Cfg64, Op>(epi, xq, wq, sx, sw, bias, out, M, N, K, ldy, s, ks);
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

// Relative throughput of one CU running a configuration's tiles, against
// the 256x256 split-ring tile (measured on MI355X at K = 3072 and 12288 on
// the DiT shapes, with the weights cold as they are at every use inside a
// model; the persistent grid runs one tile per CU at a time).  With cold
// weights 256x128 tiles beat 128x256 ones on the 768px projection and
// MLP-down (they read half the weight rows per tile), with warm ones the
// order is the other way round.
double cfg_efficiency(int cfg) {
  switch (cfg) {
    case kSplit256: return 1.0;
    case kWhole256: return 0.97;
    case k192: return 1.03;   // the next tile's first stages come during the last steps
    case kTail128x256: return 0.70;
    case k256x128: return 0.73;
    case k128: return 0.54;
    default: return 0.27;
  }
}

// Estimated time of one launch of `cfg` over an M x N x K problem, in units
// of one 256x256 tile's K loop: whole rounds of 256 tiles (a partial round
// costs as much as a full one), each as long as the tile's work over its
// efficiency, with the zero-padded stages of the ring counted.
double launch_cost(int cfg, int64_t M, int64_t N, int64_t K) {
  if (M <= 0 || N <= 0) return 0.0;
  const TileDesc& d = kCfgs[cfg];
  const int64_t tiles = ((M + d.block_m - 1) / d.block_m) * ((N + d.block_n - 1) / d.block_n);
  const int64_t rounds = (tiles + kCUs - 1) / kCUs;
  const int64_t kt = (K + d.block_k - 1) / d.block_k;
  const int64_t ring = cfg == kSplit256 || cfg == k192 ? 6 : cfg == kWhole256 ? 2
                       : cfg == kTail128x256 || cfg == k256x128 || cfg == k64 ? 3 : 4;
  const double pad = (double)((kt + ring - 1) / ring * ring) / (double)kt;
  return (double)rounds * (double)(d.block_m * d.block_n) / 65536.0 * pad / cfg_efficiency(cfg);
}

double plan_cost(int plan, int64_t M, int64_t N, int64_t K) {
  const Plan& p = kPlans[plan];
  const int64_t c = p.tail >= 0 ? main_columns(kCfgs[p.main], M, N) : 0;
  if (c == 0) return launch_cost(p.main, M, N, K);
  const int64_t nm = c * kCfgs[p.main].block_n;
  return launch_cost(p.main, M, nm, K) + launch_cost(p.tail, M, N - nm, K);
}

}  // namespace

int num_tiles() { return kNumPlans; }
const TileDesc& tile_desc(int tile) { return kCfgs[kPlans[tile].main]; }

// Shape -> plan: the cheapest plan under the cost model above (ties go to
// the earlier plan, i.e. to bigger tiles).  It reproduces the best plan of
// sweeps over all plans on the DiT shapes (M = 2304, 4096, 8192 tokens;
// K = 3072, 12288): 256x192 tiles where their count fills whole rounds
// better than 256x256 ones, 128x256 tiles for 768px shapes with about a
// hundred 256x256 tiles, 256x256 (plus the 128x256 tail) otherwise.
int select_tile(int64_t M, int64_t N, int64_t K) {
  int best = 0;
  double best_cost = plan_cost(0, M, N, K);
  for (int p = 1; p < kNumPlans; ++p) {
    const double c = plan_cost(p, M, N, K);
    if (c < best_cost * 0.999) {
      best = p;
      best_cost = c;
    }
  }
  return best;
}

// ---- K split ----
// When to split K, from sweeps on MI355X over every plan and range count
// (M = 256 ... 4096 tokens, N = 3072 / 12288, K = 3072 / 12288): a split pays
// only when the unsplit launch leaves most compute units idle and K is long.
// Its cost is the int32 slices (4 bytes per output and range, written by the
// GEMM and read back by a second pass that also writes the bf16 output) plus
// one more kernel boundary; on the 768px DiT shapes (200+ tiles) that cost
// exceeded what balancing the last round saved, e.g. 2304x3072x3072 33.6 us
// unsplit vs 50+ us in two ranges.  Measured wins: 256x3072x12288 43.4 -> 32.8
// us (8 ranges), 512x3072x12288 58.1 -> 44.1 us (4 ranges), both on 256x128
// tiles.  Rule: 256x128 tiles; split only if they number at most 64 and
// K >= 4096; double the range count while the work items stay within one
// round of 256 and each range keeps at least 768 bytes of K.
constexpr int kSplitPlan = 6;   // 256x128 main tiles

int select_splitk(int64_t M, int64_t N, int64_t K, int* tile) {
  const TileDesc& d = kCfgs[kPlans[kSplitPlan].main];
  const int64_t tiles = ((M + d.block_m - 1) / d.block_m) * ((N + d.block_n - 1) / d.block_n);
  int chunks = 1;
  if (N % 8 == 0 && tiles <= 64 && K >= 4096)
    while (tiles * chunks * 2 <= kCUs && K % (16 * chunks * 2) == 0 && K / (chunks * 2) >= 768) chunks *= 2;
  if (tile) *tile = chunks > 1 ? kSplitPlan : select_tile(M, N, K);
  return chunks;
}

template <class Op>
hipError_t launch_plan(int tile, Epilogue epi, const int8_t* xq, const int8_t* wq,
                       const float* sx, const float* sw, const uint16_t* bias, void* out,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  if (tile < 0 || tile >= kNumPlans) return hipErrorInvalidValue;
  const Plan& p = kPlans[tile];
  const int64_t c = p.tail >= 0 ? main_columns(kCfgs[p.main], M, N) : 0;
  const KSplit whole{(int)K, 1, 0};
  if (c == 0) return launch_cfg<Op>(p.main, epi, xq, wq, sx, sw, bias, out, M, N, K, N, stream, whole);
  const int64_t nm = c * kCfgs[p.main].block_n;   // channels done by the main tiles
  hipError_t e = launch_cfg<Op>(p.main, epi, xq, wq, sx, sw, bias, out, M, nm, K, N, stream, whole);
  if (e != hipSuccess) return e;
  const size_t esz = epi == Epilogue::kRawI32 ? 4 : 2;
  void* out_tail = static_cast<char*>(out) + nm * esz;
  return launch_cfg<Op>(p.tail, epi, xq, wq + nm * K, sx, sw ? sw + nm : nullptr,
                        bias ? bias + nm : nullptr, out_tail, M, N - nm, K, N, stream, whole);
}

hipError_t launch_gemm(int tile, Epilogue epi, const int8_t* xq, const int8_t* wq,
                       const float* sx, const float* sw, const uint16_t* bias, void* out,
                       int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  return launch_plan<OpI8>(tile, epi, xq, wq, sx, sw, bias, out, M, N, K, stream);
}

hipError_t launch_gemm_partials(int tile, const int8_t* xq, const int8_t* wq, int32_t* partials,
                                int64_t M, int64_t N, int64_t K, int chunks, hipStream_t stream) {
  if (tile < 0 || tile >= kNumPlans || chunks < 1 || K % (16 * chunks) != 0) return hipErrorInvalidValue;
  const KSplit ks{(int)K, chunks, M * N};
  return launch_cfg<OpI8>(kPlans[tile].main, Epilogue::kRawI32, xq, wq, nullptr, nullptr, nullptr,
                          partials, M, N, K / chunks, N, stream, ks);
}

hipError_t launch_gemm_fp8(int tile, Epilogue epi, const uint8_t* xq, const uint8_t* wq,
                           const float* sx, const float* sw, const uint16_t* bias, void* out,
                           int64_t M, int64_t N, int64_t K, hipStream_t stream) {
  return launch_plan<OpF8>(tile, epi, reinterpret_cast<const int8_t*>(xq),
                           reinterpret_cast<const int8_t*>(wq), sx, sw, bias, out, M, N, K, stream);
}

}  // namespace w8a8
