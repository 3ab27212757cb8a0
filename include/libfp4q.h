/*
 * libfp4q -- block-scaled MXFP4 linear-layer hot path for AMD MI355X (gfx950).
 *
 * C ABI.  All tensor pointers are DEVICE pointers owned by the caller; the
 * library keeps no pointer after a call returns.  Every compute call enqueues
 * its kernels on `stream` (a hipStream_t passed as void*, NULL = the default
 * stream) and returns without synchronising: a fault inside a kernel surfaces
 * at the caller's next synchronisation.  Arguments are validated on the host
 * before anything is launched; a call that returns a status other than
 * FP4Q_OK has launched nothing (except FP4Q_ERR_HIP, where a launch was
 * attempted and failed).  The library never aborts; fp4q_last_error() gives a
 * thread-local detail string for the last failing call.  Calls are reentrant
 * and thread-safe.
 *
 * Formats (sources: the MSRA FP4-training summary page, sec. 一, and the
 * outlier-dynamics page, sec. 1.1, for E2M1 on [-6, 6]; the low-precision
 * overview page, sec. 1.1, for the 8-bit exponent-only E8M0 scale; the MXFP4
 * tutorial page, sec. 4.1, for block scaling over 16..128 elements):
 *   - element: E2M1, 4-bit code = sign<<3 | magnitude code, magnitudes
 *     {0, 0.5, 1, 1.5, 2, 3, 4, 6}; two codes per byte, the element with the
 *     lower index along the block axis in the low nibble;
 *   - scale: one E8M0 byte per block, value 2^(byte-127), 0xFF = NaN;
 *     byte = clamp(floor(log2 amax) - 2, -127, 127) + 127, so the block's
 *     largest magnitude divided by the scale lies in [4, 8);
 *   - quantised operands are "K-major": [rows, K/2] code bytes and
 *     [rows, K/block] scale bytes, both dense row-major.
 *
 * Dtype codes: FP4Q_F32 = IEEE binary32, FP4Q_BF16 = bfloat16.
 * All pointers must be 16-byte aligned and every row stride (in bytes) a
 * multiple of 16, or the call returns FP4Q_ERR_ALIGNMENT; the one exception
 * is fp4q_gemm's C, which only needs its element alignment (any ld_c >= N).
 */
#ifndef LIBFP4Q_H
#define LIBFP4Q_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define FP4Q_ABI_VERSION 1

typedef enum {
    FP4Q_OK = 0,
    FP4Q_ERR_INVALID = 1,     /* null pointer, bad size, bad enum, bad block */
    FP4Q_ERR_UNSUPPORTED = 2, /* valid request this build does not implement */
    FP4Q_ERR_ALIGNMENT = 3,   /* pointer or row stride not 16-byte aligned */
    FP4Q_ERR_WORKSPACE = 4,   /* caller workspace too small */
    FP4Q_ERR_HIP = 5          /* a HIP launch or query failed */
} fp4q_status_t;

typedef enum { FP4Q_F32 = 0, FP4Q_BF16 = 1 } fp4q_dtype_t;
typedef enum { FP4Q_RNE = 0, FP4Q_SR = 1 } fp4q_round_t;
typedef enum {
    FP4Q_BLOCK_ROW = 0, /* blocks along the contiguous (last) dim  */
    FP4Q_BLOCK_COL = 1  /* blocks down the strided (first) dim     */
} fp4q_axis_t;
typedef enum { FP4Q_STE = 0, FP4Q_DGE = 1 } fp4q_grad_t;

/*
 * fp4q_quantize -- fused block amax, E8M0 scale, scale-and-round onto E2M1,
 * and nibble packing: Q(x) = s * round(x / s) (MXFP4 tutorial page, sec. 2.1)
 * with a shared power-of-two scale per block.
 *
 *   x        [rows, cols] bf16 or fp32, row stride ld_x elements (ld_x >= cols).
 *   block    16, 32, 64 or 128.
 *   axis     FP4Q_BLOCK_ROW: block j of row r = columns [j*block, (j+1)*block);
 *              codes [rows, cols/2], scales [rows, cols/block]; needs
 *              cols % block == 0.
 *            FP4Q_BLOCK_COL: block j of column c = rows [j*block, (j+1)*block);
 *              codes [cols, rows/2] and scales [cols, rows/block], i.e. the
 *              K-major quantisation of x^T; needs rows % block == 0.
 *   round    FP4Q_RNE: nearest, ties to the even code.
 *            FP4Q_SR: stochastic rounding (low-precision overview page,
 *            sec. 3.2: round up with probability equal to the fractional
 *            distance) between the two neighbouring E2M1 magnitudes
 *            lo <= m < hi of m = |x/s|, at 16-bit resolution.  With
 *            frac = (m - lo) / (hi - lo), F = floor(frac * 2^16) and u the
 *            element's 16 random bits, the magnitude becomes hi iff
 *              u + F >= 2^16        (a carry out of 16 bits),
 *            equivalently (0xFFFF - u) < F: the page's "rand < frac" with
 *            rand = (0xFFFF - u) / 2^16 and frac truncated to 16 bits, so
 *            P(hi) = F / 2^16.  This is NOT the rule u < frac * 2^16: for a
 *            given u the two disagree on up to ~90% of the u values (their
 *            probabilities agree within 2^-16).  m >= 6 gives 6; the sign is
 *            kept.  u: Philox4x32-10 (Salmon et al., SC'11) with key = seed,
 *            counter = (pos >> 3) in words 0-1 (words 2-3 zero), and 16-bit
 *            lane (pos & 7) of the output (word lane/2, low half for even
 *            lanes), pos = r*cols + c + rng_offset (the element's logical
 *            row-major index in x plus the offset).  A row shard starting at
 *            row r0 reproduces the unsharded result with
 *            rng_offset = r0*cols.  Ignored for RNE.
 *   |x/s| > 6 saturates to 6.  A block holding NaN or Inf gets scale 0xFF and
 *   all-zero codes.  The sign bit is kept (negative values that round to 0
 *   give code 0x8).
 */
fp4q_status_t fp4q_quantize(const void* x, fp4q_dtype_t x_dtype, int64_t rows, int64_t cols,
                            int64_t ld_x, int32_t block, fp4q_axis_t axis, fp4q_round_t round,
                            uint64_t seed, uint64_t rng_offset, uint8_t* codes, uint8_t* scales,
                            void* stream);

/*
 * fp4q_quantize_dual -- both block orientations of one tensor in one pass:
 * exactly the outputs of
 *   fp4q_quantize(x, ..., block, FP4Q_BLOCK_ROW, round_row, seed_row,
 *                 rng_offset, row_codes, row_scales)
 *   fp4q_quantize(x, ..., block, FP4Q_BLOCK_COL, round_col, seed_col,
 *                 rng_offset, col_codes, col_scales)
 * (layouts, rounding and random streams as there), reading x once.  A
 * training step needs an activation, a weight and an output gradient in both
 * orientations (forward GEMM operand and backward transposed operand, the
 * pages' forward/backward split of the FP4 linear layer, MSRA FP4-training
 * summary page, sec. 四), so one read serves both.
 *   rows % block == 0 and cols % block == 0; other arguments and errors as
 *   fp4q_quantize.  bf16 input runs fused; fp32 input runs as the two
 *   separate passes.
 */
fp4q_status_t fp4q_quantize_dual(const void* x, fp4q_dtype_t x_dtype, int64_t rows, int64_t cols,
                                 int64_t ld_x, int32_t block, fp4q_round_t round_row,
                                 uint64_t seed_row, fp4q_round_t round_col, uint64_t seed_col,
                                 uint64_t rng_offset, uint8_t* row_codes, uint8_t* row_scales,
                                 uint8_t* col_codes, uint8_t* col_scales, void* stream);

/*
 * fp4q_channel_mask -- builds a zero mask for fp4q_quantize_masked: bit i of
 *   mask (word i / 32, bit i % 32) is set for every i in idx[0 .. n) with
 *   0 <= i < length; all other bits of the ceil(length / 32) words are
 *   cleared.  Out-of-range indices are ignored (device data is not checked).
 *   idx int32 [n] device (may be NULL if n = 0); mask uint32 device, written.
 */
fp4q_status_t fp4q_channel_mask(const int32_t* idx, int32_t n, int64_t length, uint32_t* mask,
                                void* stream);

/*
 * fp4q_quantize_masked -- fp4q_quantize of x with the positions along the
 * block axis whose zero_mask bit is set taken as zeros (ROW: columns, COL:
 * rows; e.g. the hot channels of the outlier-dynamics page's hot-channel
 * compensation, sec. 3.1, removed from the quantised product before it is
 * formed).  Arguments and errors as fp4q_quantize, plus zero_mask: uint32
 * device bit mask over that axis (fp4q_channel_mask writes one).
 */
fp4q_status_t fp4q_quantize_masked(const void* x, fp4q_dtype_t x_dtype, int64_t rows,
                                   int64_t cols, int64_t ld_x, int32_t block, fp4q_axis_t axis,
                                   fp4q_round_t round, uint64_t seed, uint64_t rng_offset,
                                   const uint32_t* zero_mask, uint8_t* codes, uint8_t* scales,
                                   void* stream);

/*
 * fp4q_dequantize -- the QDQ partner (MXFP4 tutorial page, sec. 6.1): element
 * value(code) * 2^(byte-127), exact in fp32 and bf16 (results beyond the fp32
 * range become Inf; byte 0xFF gives NaN for the whole block).
 *   codes [rows, k/2], scales [rows, k/block] -> y [rows, k] dense, bf16/fp32.
 *   k % block == 0.
 */
fp4q_status_t fp4q_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                              int64_t k, int32_t block, void* y, fp4q_dtype_t y_dtype,
                              void* stream);

/*
 * fp4q_grad_estimate -- backward of Q: out = grad * d elementwise.
 *   FP4Q_STE: d = 1 (MXFP4 tutorial page, sec. 3.1); x may be NULL.
 *   FP4Q_DGE: the derivative of the differentiable staircase of the MSRA
 *     FP4-training summary page, sec. 二: on the E2M1 interval of width delta
 *     holding m = |x|/s (s = x's own block scale, recomputed here with the same
 *     block and axis as x's quantisation), with u = 2(m - lo)/delta - 1,
 *     d = min((1/k) |u|^(1/k - 1), clamp_max); m > 6 (saturated) gives d = 1;
 *     a block holding NaN/Inf gives NaN.
 *   x, grad, out: dense [rows, cols]; axis/block as in fp4q_quantize.
 *   k >= 1, clamp_max > 0.  The result is rounded to out_dtype once.
 */
fp4q_status_t fp4q_grad_estimate(fp4q_grad_t mode, const void* x, fp4q_dtype_t x_dtype,
                                 const void* grad, fp4q_dtype_t g_dtype, int64_t rows,
                                 int64_t cols, int32_t block, fp4q_axis_t axis, float k,
                                 float clamp_max, void* out, fp4q_dtype_t out_dtype,
                                 void* stream);

/*
 * fp4q_gemm -- FP4 x FP4 GEMM with per-block scales and fp32 accumulation
 * (the FP4 GEMMs that carry over 95% of the compute, MSRA FP4-training
 * summary page, sec. 四):
 *   C[i,j] (+)= sum_k deq(A[i,k]) * deq(B[j,k])
 *   A: a_codes [M, K/2], a_scales [M, K/32]; B: b_codes [N, K/2],
 *   b_scales [N, K/32] (both K-major, block 32, as fp4q_quantize writes them);
 *   C: [M, N] row-major with row stride ld_c elements, bf16 or fp32 (bf16 is
 *   the round-to-nearest-even of the fp32 accumulator).
 *   block must be 32 (FP4Q_ERR_UNSUPPORTED otherwise); K % 64 == 0 and
 *   K < 2^24 (larger K: FP4Q_ERR_UNSUPPORTED, since 256 rows of codes are
 *   addressed with 32-bit offsets); M, N < 2^31.
 *   accumulate = 1 adds into an fp32 C (bf16 C: FP4Q_ERR_UNSUPPORTED).
 *   M, N >= 1 are arbitrary (edge tiles are masked).  Deterministic: no
 *   atomics, no split-K.  The tile shape (256 x 256 or 128 x 384) is chosen
 *   per M, N from the device's compute-unit count; the environment variable
 *   FP4Q_GEMM_TILE=256x256 or 128x384 forces one.  With 256 x 256 tiles, more
 *   tiles than compute units and K % 1024 == 0, one persistent workgroup per
 *   compute unit walks several tiles (FP4Q_GEMM_PERSIST=0 turns this off).
 *   Every form accumulates each output over K in the same order, so all give
 *   bit-identical results.
 */
fp4q_status_t fp4q_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                        const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                        int32_t block, void* c, fp4q_dtype_t c_dtype, int64_t ld_c,
                        int32_t accumulate, void* stream);

/*
 * fp4q_gemm_dge -- the weight-gradient GEMM with the DGE gradient estimator
 * applied in its epilogue (adjacent operations around a quantisation node
 * merged, the optimisation the MXFP4 tutorial page, sec. 6.1, lists): exactly
 *   G = fp4q_gemm(A, B) into fp32, then
 *   out = fp4q_grad_estimate(FP4Q_DGE, x, G, block 32, FP4Q_BLOCK_COL, k, clamp)
 * in one kernel, without writing or re-reading G (same bits as that pair of
 * calls: the same accumulation order and the same per-element product).
 *   A, B: as fp4q_gemm (block 32); x: bf16 [M, N] dense, the weight whose
 *   estimator this is, with column blocks of 32 rows (M % 32 == 0);
 *   out: fp32 [M, N], row stride ld_out >= N, written.
 *   k >= 1, clamp_max > 0; K % 64 == 0, K < 2^24.  fp32 x:
 *   FP4Q_ERR_UNSUPPORTED.  A block of x holding NaN/Inf gives NaN.
 */
fp4q_status_t fp4q_gemm_dge(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const uint8_t* a_scales, const uint8_t* b_codes,
                            const uint8_t* b_scales, const void* x, fp4q_dtype_t x_dtype,
                            float k, float clamp_max, float* out, int64_t ld_out, void* stream);

/*
 * fp4q_gemm_quant -- a GEMM whose epilogue quantises its own bf16 output for
 * the next layer (quantisation fused into the producing kernel, the merge of
 * adjacent operations the MXFP4 tutorial page, sec. 6.1, lists): exactly
 *   C = fp4q_gemm(A, B) as bf16, then
 *   fp4q_quantize(C, bf16, block 32, FP4Q_BLOCK_ROW, FP4Q_ROUND_RNE)
 * in one kernel, without re-reading C.
 *   A, B: as fp4q_gemm (block 32; K % 64 == 0, K < 2^24).
 *   c: bf16 [M, N] with row stride ld_c >= N, written; may be NULL (then only
 *      the quantisation is written).
 *   y_codes [M, N/2], y_scales [M, N/32]: written (N % 32 == 0).
 */
fp4q_status_t fp4q_gemm_quant(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                              const uint8_t* a_scales, const uint8_t* b_codes,
                              const uint8_t* b_scales, void* c, int64_t ld_c, uint8_t* y_codes,
                              uint8_t* y_scales, void* stream);

/*
 * fp4q_hcp_workspace_bytes -- bytes of device workspace fp4q_hcp_residual_add
 * needs for these sizes.
 */
size_t fp4q_hcp_workspace_bytes(int64_t M, int64_t N, int32_t n_hot);

/*
 * fp4q_hcp_residual_add -- hot-channel compensation in the dual-kernel mode of
 * the outlier-dynamics page, sec. 3.1 (base GEMM and residual GEMM run as
 * separate kernels, then add).  Using that section's error decomposition, the
 * residual replaces the quantised operands' product on the hot channels H by
 * the bf16 operands' product:
 *   Y[i,j] += sum_{c in H} ( X[i,c] W[c,j] - Xq[i,c] Wq[c,j] )
 * computed as one bf16 GEMM with fp32 accumulation over the gathered operands
 * [X_H | Xq_H] and [W_H ; -Wq_H].
 *   x   bf16 [M, K] dense;  xq_codes/xq_scales: its ROW block-32 quantisation.
 *   w   bf16 [K, N] dense;  wq_codes/wq_scales: its COL block-32 (K-major)
 *       quantisation, [N, K/2] and [N, K/32].
 *   hot_idx  int32 [n_hot] device array of distinct channels in [0, K)
 *       (not checked: it lives on the device).  n_hot = 0 is a no-op;
 *       n_hot <= min(K, 2^20) (above 2^20: FP4Q_ERR_UNSUPPORTED).
 *   y   fp32 [M, N] dense, read and written.
 *   workspace  >= fp4q_hcp_workspace_bytes(M, N, n_hot) device bytes.
 */
fp4q_status_t fp4q_hcp_residual_add(int64_t M, int64_t N, int64_t K, const void* x,
                                    const uint8_t* xq_codes, const uint8_t* xq_scales,
                                    const void* w, const uint8_t* wq_codes,
                                    const uint8_t* wq_scales, const int32_t* hot_idx,
                                    int32_t n_hot, float* y, void* workspace,
                                    size_t workspace_bytes, void* stream);

/*
 * fp4q_hcp_residual_add_noalloc -- fp4q_hcp_residual_add without a caller
 * workspace, for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc).  The
 * same kernels and results as fp4q_hcp_residual_add (bit for bit); the
 * gathered hot operands go to a library-owned device array of
 * FP4Q_HCP_NOALLOC_MAX_BYTES (64 MiB) instead, which each GPU the library
 * runs on holds until the process ends.  This call allocates nothing.
 *   Arguments and limits as fp4q_hcp_residual_add (minus the workspace).
 *   fp4q_hcp_workspace_bytes(M, N, n_hot) must not exceed
 *   FP4Q_HCP_NOALLOC_MAX_BYTES, else FP4Q_ERR_WORKSPACE (nothing launched);
 *   the 16384 x 13824 layer with 461 hot channels needs 56 MB.
 *   Every call on one GPU shares that GPU's array: calls that overlap on one
 *   GPU (two streams, two threads) race and may corrupt each other's results;
 *   calls ordered on one stream are safe.  The array's contents are not kept
 *   between calls (every call writes what it reads).
 */
#define FP4Q_HCP_NOALLOC_MAX_BYTES ((size_t)64 << 20)
fp4q_status_t fp4q_hcp_residual_add_noalloc(int64_t M, int64_t N, int64_t K, const void* x,
                                            const uint8_t* xq_codes, const uint8_t* xq_scales,
                                            const void* w, const uint8_t* wq_codes,
                                            const uint8_t* wq_scales, const int32_t* hot_idx,
                                            int32_t n_hot, float* y, void* stream);

/*
 * fp4q_gemm_hcp -- hot-channel compensation in the single-kernel mode of the
 * outlier-dynamics page, sec. 3.1 (the hot-channel terms are computed inside
 * the main GEMM instead of by a second kernel):
 *   Y[i,j] = sum_k Xq[i,k] Wq[k,j]
 *          + sum_{c in H} ( X[i,c] W[c,j] - Xq[i,c] Wq[c,j] )
 * i.e. fp4q_gemm into an fp32 Y followed by fp4q_hcp_residual_add, in one
 * GEMM kernel: its FP4 K loop over all K, then a bf16 K loop over the
 * gathered [X_H | Xq_H] and [W_H ; -Wq_H] into the same fp32 accumulators.
 * Y is written once and never read (no fp32 read-modify-write of Y).
 *   x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx, n_hot, workspace:
 *       as fp4q_hcp_residual_add (block 32 quantisations: X ROW, W COL).
 *   y   fp32 [M, N], row stride ld_y >= N elements, written.
 *   K % 64 == 0 and K < 2^24 as fp4q_gemm; n_hot <= min(K, 2^20).
 *   n_hot = 0: Y is the plain FP4 GEMM (x, w, hot_idx, workspace may be NULL).
 *   Summation order differs from the two-call form (one accumulator), so
 *   results agree with it to fp32 rounding, not bit for bit.
 */
fp4q_status_t fp4q_gemm_hcp(int64_t M, int64_t N, int64_t K, const void* x,
                            const uint8_t* xq_codes, const uint8_t* xq_scales, const void* w,
                            const uint8_t* wq_codes, const uint8_t* wq_scales,
                            const int32_t* hot_idx, int32_t n_hot, float* y, int64_t ld_y,
                            void* workspace, size_t workspace_bytes, void* stream);

/*
 * fp4q_gemm_hcp_split -- hot-channel compensation, the "split" reading of
 * the outlier-dynamics page, sec. 3.1-3.2: the hot channels H are removed
 * from the quantised product (xq and wq come from fp4q_quantize_masked with
 * H zeroed: X's columns, W's rows) and their bf16 product is added:
 *   Y[i,j] = sum_k Xq'[i,k] Wq'[k,j] + sum_{c in H} X[i,c] W[c,j]
 * in one GEMM kernel (FP4 K loop, then a bf16 K loop of depth |H| padded to
 * 32).  Arguments and limits as fp4q_gemm_hcp; y fp32 [M, N] (row stride
 * ld_y) is written.
 */
fp4q_status_t fp4q_gemm_hcp_split(int64_t M, int64_t N, int64_t K, const void* x,
                                  const uint8_t* xq_codes, const uint8_t* xq_scales,
                                  const void* w, const uint8_t* wq_codes,
                                  const uint8_t* wq_scales, const int32_t* hot_idx,
                                  int32_t n_hot, float* y, int64_t ld_y, void* workspace,
                                  size_t workspace_bytes, void* stream);

/*
 * fp4q_quantize_2d -- two-dimensional block scaling: one E8M0 scale per
 * 32 x 32 square of x (the outlier-dynamics page, sec. 4.1, scales the
 * backward pass's operands in 2D blocks; MXFP4's 32-element block is used in
 * both directions, the granularity at which the GEMM takes scales along K).
 * Each square is quantised as one block (scale from the square's largest
 * |x|, elements rounded as fp4q_quantize rounds them) and the same codes are
 * written in both layouts:
 *   row_codes [rows, cols/2], row_scales [rows, cols/32]: the ROW layout,
 *       each square's scale repeated on its 32 rows (a GEMM operand that
 *       contracts over columns);
 *   col_codes [cols, rows/2], col_scales [cols, rows/32]: the COL (K-major)
 *       layout, each square's scale repeated on its 32 columns (the operand
 *       that contracts over rows).
 * Dequantised, the two are one matrix and its transpose, so a weight enters
 * the forward GEMM and the data-gradient GEMM with the same values.
 *   x bf16 [rows, cols], row stride ld_x >= cols (multiple of 8 elements);
 *   rows % 32 == 0, cols % 32 == 0; all pointers 16-byte aligned.
 *   round FP4Q_RNE or FP4Q_SR; SR draws element (r, c) from counter
 *   r*cols + c + rng_offset of seed's stream, as fp4q_quantize does.
 *   A square holding Inf or NaN gets scale 0xFF and zero codes.
 */
fp4q_status_t fp4q_quantize_2d(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                               fp4q_round_t round, uint64_t seed, uint64_t rng_offset,
                               uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                               uint8_t* col_scales, void* stream);

/*
 * fp4q_quantize_2d_tile -- fp4q_quantize_2d with the square side as an
 * argument: tile = 32 is fp4q_quantize_2d; tile = 16 gives the 16 x 16
 * backward blocks that the outlier-dynamics page's configuration names
 * (sec. 4.2), one E8M0 scale per 16 x 16 square (scale from the square's
 * largest |x|, elements rounded as fp4q_quantize rounds them, SR counters
 * r*cols + c + rng_offset), written in the same two layouts with block 16:
 *   row_codes [rows, cols/2], row_scales [rows, cols/16];
 *   col_codes [cols, rows/2], col_scales [cols, rows/16].
 * Each layout dequantises with fp4q_dequantize(..., block = 16).  The
 * hardware GEMM takes one scale per 32 elements, so the 16 x 16 form is a
 * quantise/dequantise form; 32 x 32 is the GEMM-feeding one.
 *   tile 16 or 32 (else FP4Q_ERR_INVALID); other arguments, limits and errors
 *   as fp4q_quantize_2d (rows % 32 == 0, cols % 32 == 0 for both tiles).
 */
fp4q_status_t fp4q_quantize_2d_tile(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                    int32_t tile, fp4q_round_t round, uint64_t seed,
                                    uint64_t rng_offset, uint8_t* row_codes, uint8_t* row_scales,
                                    uint8_t* col_codes, uint8_t* col_scales, void* stream);

/*
 * fp4q_quantize_rht -- random Hadamard transform, then block-32 quantisation
 * (the recipe on the outlier-dynamics page, sec. 4.1, transforms the
 * backward pass's operands before quantising them).  Along the block axis,
 * each group of 32 values x (the group of one quantisation block) becomes
 *   y = 2^-2.5 * H32 * D * x,
 * with H32 the natural-order (Sylvester) Hadamard matrix, entries
 * (-1)^popcount(i & j), and D = diag(-1 where the sign bit of the position is
 * set, else +1), so 2^-2.5 * H32 is orthogonal: a GEMM whose two operands are
 * transformed along their shared contraction axis with the same sign mask
 * approximates the untransformed product (no correction factor).  y is
 * evaluated in fp32 (five levels of butterflies (a, b) -> (a + b, a - b),
 * then the product by 2^-2.5 rounded to fp32), so each value is within
 * 8 * 2^-24 * 2^-2.5 * sum|x| (+ 2^-149) of the exact y; the fp32 values are
 * then quantised exactly as fp4q_quantize quantises an fp32 tensor (block
 * 32, same layouts, rounding and random counters r*cols + c + rng_offset).
 * The codes and scales are therefore those of the exact y wherever that
 * bound crosses no rounding or scale boundary (nearly every element), and
 * one of the two neighbouring results elsewhere; the evaluation order is
 * fixed, so results are deterministic.
 *   x      bf16 [rows, cols], row stride ld_x >= cols (multiple of 8).
 *   axis   FP4Q_BLOCK_ROW: groups along columns, cols % 32 == 0; codes
 *            [rows, cols/2], scales [rows, cols/32].
 *          FP4Q_BLOCK_COL: groups along rows, rows % 32 == 0, cols even;
 *            codes [cols, rows/2], scales [cols, rows/32] (K-major).
 *   signs  uint32 device bit mask over the block axis (bit i of word i/32
 *          negates position i; cols bits for ROW, rows bits for COL),
 *          4-byte aligned; the caller draws it (e.g. once per layer) and
 *          passes the same mask for both operands of a GEMM.
 *   round, seed, rng_offset as fp4q_quantize.  x, codes, scales 16-byte
 *   aligned.  A group holding Inf or NaN (or overflowing fp32) gets scale
 *   0xFF and zero codes.
 */
fp4q_status_t fp4q_quantize_rht(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                fp4q_axis_t axis, const uint32_t* signs, fp4q_round_t round,
                                uint64_t seed, uint64_t rng_offset, uint8_t* codes,
                                uint8_t* scales, void* stream);

/*
 * fp4q_occ_quantize -- outlier clamping and compensation (the MSRA
 * FP4-training summary page, sec. 三: the largest 1% of activation values
 * are clamped to the 99th-percentile threshold before quantisation, and what
 * the clamp removes is kept in a sparse matrix handled in high precision;
 * sec. 六: FP4 main path plus a higher-precision sparse path).  For the bf16
 * x [rows, cols] with n = rows*cols elements:
 *   T = the j-th smallest |x| over the whole tensor, j = ceil(quantile * n)
 *       clamped to [1, n] (an order statistic of the bf16 magnitudes; NaN
 *       ranks above every number), written to *threshold as bf16 magnitude
 *       bits if threshold is not NULL;
 *   outliers: the elements whose |x| ranks above T (with a finite T this
 *       includes NaN; with a NaN T there are none);
 *   clamp(x) = sign(x) * T on outliers, x elsewhere (exact in bf16);
 *   codes, scales: fp4q_quantize(clamp(x), BF16, rows, cols, cols, 32,
 *       FP4Q_BLOCK_ROW, round, seed, rng_offset) exactly (ROW layout);
 *   the residual R = x - clamp(x) in CSR: row_ptr int64 [rows + 1],
 *       col_idx int32 and vals fp32 [row_ptr[rows]], columns ascending within
 *       a row, each value the fp32 rounding of the exact difference.
 * The number of outliers is at most n - j = fp4q_occ_max_nnz(rows, cols,
 * quantile); nnz_cap (the length of col_idx and vals) must be at least that.
 *   quantile in (0, 1]; cols % 32 == 0; n < 2^32; ld_x >= cols, ld_x % 8 == 0.
 *   workspace >= fp4q_occ_workspace_bytes(rows, cols) device bytes (16-byte
 *   aligned; holds a 32768-bin histogram, row counts and a 1-bit outlier
 *   mask; contents not kept).  x, codes, scales 16-byte aligned; row_ptr
 *   8-byte, col_idx and vals 4-byte aligned.
 */
int64_t fp4q_occ_max_nnz(int64_t rows, int64_t cols, double quantile);
size_t fp4q_occ_workspace_bytes(int64_t rows, int64_t cols);
fp4q_status_t fp4q_occ_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                double quantile, fp4q_round_t round, uint64_t seed,
                                uint64_t rng_offset, uint8_t* codes, uint8_t* scales,
                                int64_t* row_ptr, int32_t* col_idx, float* vals, int64_t nnz_cap,
                                uint16_t* threshold, void* workspace, size_t workspace_bytes,
                                void* stream);

/*
 * fp4q_occ_spmm -- the compensation product of the same passage: for the
 * residual R [M, K] in the CSR form fp4q_occ_quantize writes,
 *   Y[i, :] += sum over row i's entries, in CSR order, of R[i,k] * W[k, :]
 * in fp32 (fused multiply-adds from zero, then one add into Y); rows without
 * entries leave Y untouched.  Y = Xq Wq (fp4q_gemm of the clamped
 * activation, fp32 out) + R W is the compensated product.
 *   w  bf16 [K, N], row stride ld_w >= N (ld_w % 8 == 0);
 *   y  fp32 [M, N], row stride ld_y >= N (ld_y % 4 == 0), read and written;
 *   N % 8 == 0; column indices must lie in [0, K) (device data, not checked).
 *   w, y 16-byte aligned; row_ptr 8-byte, col_idx and vals 4-byte aligned.
 */
fp4q_status_t fp4q_occ_spmm(int64_t M, int64_t N, int64_t K, const int64_t* row_ptr,
                            const int32_t* col_idx, const float* vals, const void* w,
                            int64_t ld_w, float* y, int64_t ld_y, void* stream);

/*
 * fp4q_hot_channels -- the choice of the hot channels H (outlier-dynamics
 * page, sec. 4.1: the top 9% of channels by quantisation error are kept in
 * high precision, the choice refreshed every 1000 steps).  The error of
 * channel c of X is
 *   e_c = sum_i ( X[i,c] - deq(Q(X))[i,c] )^2
 * with Q the ROW block-32 nearest-even quantisation that fp4q_quantize
 * gives X (a block holding Inf or NaN dequantises to NaN, so e_c is NaN).
 * The n_hot channels of largest e_c are written to hot_idx in ascending
 * index order, ready for fp4q_quantize_masked / fp4q_channel_mask and the
 * hot-channel GEMMs.  Ranking: NaN above every number, equal errors to the
 * lower index.  e_c is summed in fp32 (squares rounded, a fixed order that
 * does not depend on scheduling), so the choice is deterministic run to run.
 *   x        bf16 [rows, cols], row stride ld_x >= cols (ld_x % 8 == 0),
 *            16-byte aligned; read only.
 *   cols % 32 == 0, cols <= 16384 (above: FP4Q_ERR_UNSUPPORTED);
 *   0 <= n_hot <= cols.
 *   hot_idx  int32 [n_hot], written (may be NULL when n_hot = 0).
 *   err      fp32 [cols], e_c written; NULL to skip it.
 *   workspace >= fp4q_hot_channels_workspace_bytes(rows, cols) device bytes,
 *            16-byte aligned; caller-owned, contents not kept.
 */
size_t fp4q_hot_channels_workspace_bytes(int64_t rows, int64_t cols);
fp4q_status_t fp4q_hot_channels(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                int32_t n_hot, int32_t* hot_idx, float* err, void* workspace,
                                size_t workspace_bytes, void* stream);

/*
 * fp4q_set_next_launch -- options for the next kernel that this thread
 * launches through the library (the first kernel of the next entry point
 * called, for entry points that launch several).  With any option given,
 * that kernel is dispatched with hipExtLaunchKernel:
 *   start_event, stop_event  hipEvent_t (as void*), created and owned by
 *            the caller, either may be NULL: recorded by the dispatch itself
 *            at the kernel's start and end, so hipEventElapsedTime of the
 *            pair is that kernel's own duration, as a kernel trace reports
 *            it (separate hipEventRecord calls around the entry point would
 *            add the marker packets' queue time).
 *   flags    0, or FP4Q_LAUNCH_ANY_ORDER: the kernel may start before the
 *            work queued earlier on its stream has finished (its dispatch
 *            carries no barrier).  The caller guarantees that the kernel
 *            reads nothing that earlier, unfinished work writes and writes
 *            nothing that work reads.  A later launch without the flag (the
 *            default) waits for everything before it, this kernel included.
 * The options are used once: the launch that takes them clears them.  An
 * entry point that fails before launching leaves them pending; calling with
 * (NULL, NULL, 0) clears them.  Thread-local: other threads' launches are
 * not affected.
 * Errors: FP4Q_ERR_INVALID for unknown flag bits (nothing is set).
 */
#define FP4Q_LAUNCH_ANY_ORDER 1u
fp4q_status_t fp4q_set_next_launch(void* start_event, void* stop_event, uint32_t flags);

const char* fp4q_status_string(fp4q_status_t s);
const char* fp4q_last_error(void);
int32_t fp4q_abi_version(void);

#ifdef __cplusplus
}
#endif

#endif /* LIBFP4Q_H */
