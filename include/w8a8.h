/*
 * w8a8.h — C ABI of the MI355X (gfx950) fused W8A8 linear library, libw8a8.so.
 *
 * The operation is the one in the abstract of "Realizing Native INT8 Compute
 * for Diffusion Transformers on Consumer GPUs: A Fused INT8 GEMM Kernel for
 * Ideogram 4.0" (arXiv 2606.14598): activations are quantized to int8 per
 * token, weights per (output) channel, the product is accumulated
 * int8 x int8 -> int32 on the matrix cores, and the per-token x per-channel
 * dequantization plus the bias are folded into the GEMM epilogue, which
 * writes bf16.
 *
 * Conventions shared by every entry point
 *   - All tensors are dense, row-major, in device memory (hipMalloc'd or a
 *     torch device tensor); bf16 values are passed as their uint16_t bits.
 *   - X is [M,K] (one row per token), W is [N,K] (one row per output channel,
 *     the torch nn.Linear layout), Y is [M,N].
 *   - The caller owns every buffer.  The library allocates no device memory,
 *     keeps no pointer after returning and holds no mutable state; it is
 *     thread-safe.
 *   - Work is enqueued asynchronously on `stream` (0 = the null stream);
 *     results are valid once that stream has been synchronised.
 *   - Arguments are validated before anything is launched; on any error
 *     nothing is launched and no output byte is written.  Shapes are checked
 *     first: an empty input (M == 0, or N == 0 for the weight quantizer) is
 *     then a no-op that returns W8A8_OK without looking at the pointers.
 *   - Inputs must be finite.  NaN/Inf inputs are outside the contract and not
 *     checked on the hot path.
 *   - Shape contract: 16 <= K, K % 16 == 0; N >= 1; M >= 0.  The GEMM entry
 *     points also require K <= W8A8_MAX_K, the largest K for which a sum of
 *     K products of codes in [-127, 127] cannot overflow int32.
 *   - Alignment contract: X, W, Xq and Wq 16-byte aligned; scales 4-byte
 *     aligned; Y and bias 2-byte aligned; int32 accumulators 4-byte aligned.
 */
#ifndef W8A8_H_
#define W8A8_H_

#include <stddef.h>
#include <stdint.h>
#include <hip/hip_runtime_api.h>

#ifdef __cplusplus
extern "C" {
#endif

/* floor((2^31 - 1) / 127^2): sums of this many +-127*127 products fit int32. */
#define W8A8_MAX_K 133144

typedef enum {
  W8A8_OK = 0,
  W8A8_ERR_NULL = 1,   /* a required pointer is NULL */
  W8A8_ERR_SHAPE = 2,  /* M, N or K outside the shape contract */
  W8A8_ERR_ALIGN = 3,  /* a pointer breaks the alignment contract */
  W8A8_ERR_LAUNCH = 4, /* the HIP runtime rejected a launch (wrong device, no device, ...) */
  W8A8_ERR_ARG = 5,    /* any other invalid argument (e.g. an unknown tile id) */
  W8A8_ERR_SCRATCH = 6, /* more scratch than the no-allocation entry point holds */
  /* Not statuses: these two make every int32 value a valid w8a8_status, so
   * that C++ code may hold and compare any value a C caller passes (without
   * them a value outside 0..7 is undefined behaviour in C++). */
  W8A8_STATUS_RANGE_MIN_ = -2147483647 - 1,
  W8A8_STATUS_RANGE_MAX_ = 2147483647
} w8a8_status;

/* Static, NUL-terminated description of a status code. */
const char *w8a8_status_str(w8a8_status s);

/*
 * Per-output-channel weight quantization (offline, once per layer).
 * For each row n of w [N,K] (bf16 bits):
 *   amax = max_k |w[n,k]|,  w_scale[n] = fl32(amax / 127),
 *   wq[n,k] = clamp(rne(fl32(w[n,k] / w_scale[n])), -127, 127),
 * an all-zero row gives w_scale[n] = 0 and wq[n,:] = 0.
 * Abstract: weights are quantized and their per-channel scale is folded into
 * the epilogue.  Outputs: wq int8 [N,K], w_scale fp32 [N].
 */
w8a8_status w8a8_quantize_weight(const uint16_t *w, int64_t N, int64_t K,
                                 int8_t *wq, float *w_scale, hipStream_t stream);

/*
 * Per-token activation quantization (every forward).  Same row rule as
 * w8a8_quantize_weight applied to each row m of x [M,K]:
 * outputs xq int8 [M,K] and x_scale fp32 [M].
 * Abstract: activations are quantized per token.
 */
w8a8_status w8a8_quantize_act(const uint16_t *x, int64_t M, int64_t K,
                              int8_t *xq, float *x_scale, hipStream_t stream);

/*
 * The fp8 variant of the method (OCP e4m3 codes instead of int8; the pages
 * weigh the int8 path against fp8 alternatives, here the same kernels run
 * both on one GPU).  Codes are uint8 bit patterns of e4m3 (1 sign, 4
 * exponent bits with bias 7, 3 mantissa bits; largest value 448).
 *   quantize:  s = fl32(amax / 448), q = e4m3(fl32(v / s)) (nearest, ties to
 *              even, saturating at +-448); an all-zero row gives s = 0, q = 0.
 *   GEMM:      acc[m,n] = sum_k x[m,k] * w[n,k] accumulated in fp32 on the
 *              matrix cores (v_mfma_f32_32x32x64_f8f6f4).  The products are
 *              exact; each instruction adds a block of 64 of them at the
 *              hardware's own internal precision and order, which the ISA
 *              does not document, so the sums are not those of sequential
 *              fp32 additions and carry no bound of the form
 *              gamma_K * sum |x w|.  Checked against exact sums to the same
 *              output tolerance as the int8 path.
 *   linear:    the same epilogue as w8a8_linear on the fp32 accumulators.
 * Same shape, alignment and error contracts as the int8 entry points; the
 * raw entry writes fp32 accumulators.
 */
w8a8_status w8a8_quantize_weight_fp8(const uint16_t *w, int64_t N, int64_t K, uint8_t *wq,
                                     float *w_scale, hipStream_t stream);
w8a8_status w8a8_quantize_act_fp8(const uint16_t *x, int64_t M, int64_t K, uint8_t *xq,
                                  float *x_scale, hipStream_t stream);
w8a8_status w8a8_linear_fp8(const uint8_t *xq, const float *x_scale, const uint8_t *wq,
                            const float *w_scale, const uint16_t *bias, uint16_t *y,
                            int64_t M, int64_t N, int64_t K, hipStream_t stream);
w8a8_status w8a8_linear_fp8_tile(const uint8_t *xq, const float *x_scale, const uint8_t *wq,
                                 const float *w_scale, const uint16_t *bias, uint16_t *y,
                                 int64_t M, int64_t N, int64_t K, int tile, hipStream_t stream);
w8a8_status w8a8_gemm_f32_fp8(const uint8_t *xq, const uint8_t *wq, float *acc,
                              int64_t M, int64_t N, int64_t K, hipStream_t stream);
w8a8_status w8a8_gemm_f32_fp8_tile(const uint8_t *xq, const uint8_t *wq, float *acc,
                                   int64_t M, int64_t N, int64_t K, int tile, hipStream_t stream);

/*
 * Row-wise dequantization back to bf16 (the slow path's first step):
 *   out[r,k] = bf16_rne( fl32( float(q[r,k]) * scale[r] ) )
 * for q int8 [R,K] and scale fp32 [R]; out is bf16 [R,K].
 * Abstract: the shipped int8 forward this work replaces quantizes
 * weights and activations and then immediately dequantizes them to bf16 for a
 * bf16 matrix multiply.  Provided so that path can be measured against the
 * fused GEMM; it is not part of the fused path.  Shape contract as above
 * (16 <= K, K % 16 == 0, R >= 0; R == 0 is a no-op); q and out 16-byte
 * aligned, scale 4-byte aligned.
 */
w8a8_status w8a8_dequantize_rows(const int8_t *q, const float *scale, int64_t R, int64_t K,
                                 uint16_t *out, hipStream_t stream);

/*
 * Fused W8A8 linear: int8 GEMM with the dequant + bias epilogue.
 *   acc[m,n] = sum_k xq[m,k] * wq[n,k]                 (exact, int32)
 *   y[m,n]   = bf16_rne( fl32( fl32( fl32(float(acc[m,n]) * x_scale[m])
 *                                    * w_scale[n] ) + float(bias[n]) ) )
 * Each fp32 operation is rounded separately (no fused multiply-add), so y is
 * a deterministic function of the inputs.  bias may be NULL (treated as 0).
 * Abstract: int8 x int8 -> int32 on the matrix cores, per-token x per-channel
 * dequantization and bias folded into the epilogue, bf16 out.
 * Inputs xq [M,K], x_scale [M], wq [N,K], w_scale [N], bias [N]; output y [M,N].
 */
w8a8_status w8a8_linear(const int8_t *xq, const float *x_scale, const int8_t *wq,
                        const float *w_scale, const uint16_t *bias, uint16_t *y,
                        int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * Fused W8A8 linear with GELU in the epilogue (the up-projection of a
 * transformer MLP):
 *   y[m,n] = bf16_rne( gelu( fl32 value of w8a8_linear above ) ),
 *   gelu(v) = v * Phi(v) (exact erf definition), evaluated in fp32 with a
 *   relative error below 3e-5 (below 1e-5 where |gelu| > 1e-6).
 * Abstract: the per-token x per-channel dequantization and the bias are
 * folded into the GEMM epilogue; the activation that follows the linear is
 * folded in the same way, so the pre-activation never reaches memory.  Not
 * bit-reproducible against an fp64 GELU: compare with a tolerance.  Same
 * arguments, contracts and errors as w8a8_linear / w8a8_linear_tile.
 */
w8a8_status w8a8_linear_gelu(const int8_t *xq, const float *x_scale, const int8_t *wq,
                             const float *w_scale, const uint16_t *bias, uint16_t *y,
                             int64_t M, int64_t N, int64_t K, hipStream_t stream);
w8a8_status w8a8_linear_gelu_tile(const int8_t *xq, const float *x_scale, const int8_t *wq,
                                  const float *w_scale, const uint16_t *bias, uint16_t *y,
                                  int64_t M, int64_t N, int64_t K, int tile, hipStream_t stream);

/*
 * Diagnostic entry: the same GEMM main loop, storing the raw int32
 * accumulators acc [M,N] instead of running the epilogue.
 * Abstract: the int8 x int8 -> int32 accumulation is checked bit for bit.
 */
w8a8_status w8a8_gemm_i32(const int8_t *xq, const int8_t *wq, int32_t *acc,
                          int64_t M, int64_t N, int64_t K, hipStream_t stream);

/*
 * Per-shape tile selection (the abstract tunes its kernel for each GEMM shape;
 * here a fixed table chosen from measurements).  w8a8_num_tiles() is the number of
 * compiled tile configurations; w8a8_tile_info() describes one (block rows of
 * X, block rows of W, K bytes per stage, threads; any pointer may be NULL);
 * w8a8_select_tile() returns the id w8a8_linear would use for a shape.
 */
int w8a8_num_tiles(void);
w8a8_status w8a8_tile_info(int tile, int *block_m, int *block_n, int *block_k, int *threads);
int w8a8_select_tile(int64_t M, int64_t N, int64_t K);

/*
 * w8a8_linear / w8a8_gemm_i32 with an explicit tile id (tile < 0 selects as
 * the plain entry points do).  Every tile gives bit-identical results; these
 * exist for tests and tile sweeps.  An unknown id returns W8A8_ERR_ARG.
 */
w8a8_status w8a8_linear_tile(const int8_t *xq, const float *x_scale, const int8_t *wq,
                             const float *w_scale, const uint16_t *bias, uint16_t *y,
                             int64_t M, int64_t N, int64_t K, int tile, hipStream_t stream);
w8a8_status w8a8_gemm_i32_tile(const int8_t *xq, const int8_t *wq, int32_t *acc,
                               int64_t M, int64_t N, int64_t K, int tile, hipStream_t stream);

/*
 * K-split fused linear, for shapes whose output tiles are too few to occupy
 * every compute unit (few tokens and a long K, e.g. the down-projection of a
 * transformer MLP over a small batch).  Same result, bit for bit, as
 * w8a8_linear (or w8a8_linear_gelu when `gelu` is non-zero): the K reduction
 * of each output tile is cut into `splits` equal ranges, each range's exact
 * int32 sums are written to the caller's workspace, and a second pass adds
 * the ranges (exactly, in int32) and applies the same fp32 dequantization,
 * bias (and GELU) epilogue, rounded to bf16.
 * Abstract: int8 x int8 -> int32 on the matrix cores, per-token x
 * per-channel dequantization and bias folded into the epilogue; the pages'
 * GEMM is tuned per shape, and splitting K is this library's answer for
 * shapes with few output tiles.
 *   splits <= 0: chosen by the library's cost model (w8a8_select_splitk);
 *   splits == 1: the plain fused path, no workspace needed;
 *   splits > 1: requires N % 8 == 0, K % (16 * splits) == 0 (else
 *                W8A8_ERR_SHAPE), splits <= 64, y and workspace 16-byte
 *                aligned, and workspace_bytes >=
 *                w8a8_linear_splitk_workspace(M, N, splits) (else W8A8_ERR_ARG).
 *   tile < 0: automatic; else a tile id as for w8a8_linear_tile (its main
 *   tiles are used; W8A8_ERR_ARG if unknown).
 * The workspace (device memory the caller owns, splits * M * N int32) is
 * written and read only by this call's kernels, in stream order; calls that
 * share a workspace must be ordered on one stream.
 */
int w8a8_select_splitk(int64_t M, int64_t N, int64_t K, int *tile);
size_t w8a8_linear_splitk_workspace(int64_t M, int64_t N, int splits);
w8a8_status w8a8_linear_splitk(const int8_t *xq, const float *x_scale, const int8_t *wq,
                               const float *w_scale, const uint16_t *bias, uint16_t *y,
                               int64_t M, int64_t N, int64_t K, int splits, int tile, int gelu,
                               void *workspace, size_t workspace_bytes, hipStream_t stream);

/*
 * w8a8_linear_splitk for callers that cannot allocate device memory (code
 * under HIP graph capture, tight serving loops, harnesses that forbid
 * hipMalloc): the same arguments and result without the workspace.  The int32
 * slices live in a library-owned array of W8A8_NOALLOC_SCRATCH_BYTES (32 MiB)
 * in each GPU's memory, held from the library's load until the process ends;
 * its device address is looked up (hipGetSymbolAddress) on the first call on
 * each device, with that device current.  The call allocates nothing.
 * Every call on one GPU uses that GPU's one array: calls that may overlap on
 * one GPU (different streams, or different host threads without ordering)
 * race on it and must be serialized by the caller; calls in order on one
 * stream are safe.  No state carries from one call to the next (each slice
 * element is written before it is read).  A request whose split needs more
 * than W8A8_NOALLOC_SCRATCH_BYTES (splits * M * N * 4 bytes, splits as
 * resolved when `splits` <= 0) returns W8A8_ERR_SCRATCH before anything is
 * launched.  The current device must be the one `stream` belongs to.
 */
#define W8A8_NOALLOC_SCRATCH_BYTES (32 * 1024 * 1024)
w8a8_status w8a8_linear_splitk_noalloc(const int8_t *xq, const float *x_scale, const int8_t *wq,
                                       const float *w_scale, const uint16_t *bias, uint16_t *y,
                                       int64_t M, int64_t N, int64_t K, int splits, int tile,
                                       int gelu, hipStream_t stream);

/*
 * Diagnostic: the throughput ceiling of w8a8_linear's inner loop on this GPU,
 * on the caller's codes.  The int8 matrix cores run at a power-limited clock
 * that depends on the operand values, so the GEMM's rate is best read against
 * what the same instructions sustain on the same data.  This runs the GEMM's
 * K step exactly (the 256x192 tile's eight wavefronts, fragment reads from
 * LDS one K step ahead of the int8 MFMAs) on one 128-byte K stage of xq
 * [M,K] and wq [N,K] per workgroup, staged in LDS once and looped over
 * `iters` times, with no memory traffic, barriers or epilogue in the loop:
 * 256 workgroups of 512 threads, each 49152 * iters MFMAs of
 * 32x32x32 int8 (65536 int8 operations each).  Time it with events on
 * `stream`.
 * Workgroup g takes rows m0 = (g mod floor(M/256)) * 256 of xq,
 * n0 = (floor(g / floor(M/256)) mod floor(N/192)) * 192 of wq and the K stage
 * k0 = (g mod floor(K/128)) * 128; its eight wavefronts write the sums of
 * their int32 accumulators to sink[g*8 .. g*8+7] (int64, device memory,
 * 2048 entries), which add up to iters * sum over k in the stage of
 * (sum of xq[m0..m0+255, k]) * (sum of wq[n0..n0+191, k]).
 * Requires 256 <= M, 192 <= N, 128 <= K <= W8A8_MAX_K, K % 16 == 0 and
 * 1 <= iters <= 2^40; xq, wq 16-byte and sink 8-byte aligned.  Not part of
 * the fused path; it exists so measurements can be put against the chip's
 * power-limited matrix-core rate.
 */
w8a8_status w8a8_mfma_ceiling(const int8_t *xq, const int8_t *wq, int64_t M, int64_t N, int64_t K,
                              int64_t iters, int64_t *sink, hipStream_t stream);

#ifdef __cplusplus
}
#endif

#endif /* W8A8_H_ */
