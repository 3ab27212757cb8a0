// libfp4q C ABI: host-side validation, status reporting and kernel dispatch.
// Every entry point checks its arguments before touching the device and
// launches nothing when it returns an error other than FP4Q_ERR_HIP.
#include <cmath>
#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include "../../include/libfp4q.h"
#include "fp4q_internal.h"

namespace fp4q {
thread_local NextLaunch g_next_launch = {nullptr, nullptr, 0u, false};
}

namespace {

thread_local char g_err[512] = "";

fp4q_status_t fail(fp4q_status_t s, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
fp4q_status_t fail(fp4q_status_t s, const char* fmt, ...) {
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(g_err, sizeof g_err, fmt, ap);
    va_end(ap);
    return s;
}

fp4q_status_t hip_status(hipError_t e, const char* where) {
    if (e == hipSuccess) return FP4Q_OK;
    return fail(FP4Q_ERR_HIP, "%s: %s", where, hipGetErrorString(e));
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }
bool valid_block(int32_t b) { return b == 16 || b == 32 || b == 64 || b == 128; }
bool valid_dtype(int d) { return d == FP4Q_F32 || d == FP4Q_BF16; }
int64_t esize(int d) { return d == FP4Q_BF16 ? 2 : 4; }

static_assert(fp4q::kHcpStaticScratchBytes == FP4Q_HCP_NOALLOC_MAX_BYTES,
              "the header states the size of the library-owned hot-channel scratch");

// Index arithmetic inside the streaming kernels is 32-bit over 8-element
// chunks; element counts up to 2^33 are accepted.
constexpr int64_t kMaxElems = (int64_t)1 << 33;

}  // namespace

extern "C" {

int32_t fp4q_abi_version(void) { return FP4Q_ABI_VERSION; }

const char* fp4q_last_error(void) { return g_err; }

fp4q_status_t fp4q_set_next_launch(void* start_event, void* stop_event, uint32_t flags) {
    if (flags & ~(uint32_t)FP4Q_LAUNCH_ANY_ORDER)
        return fail(FP4Q_ERR_INVALID, "set_next_launch: unknown flags 0x%x", flags);
    fp4q::g_next_launch = fp4q::NextLaunch{(hipEvent_t)start_event, (hipEvent_t)stop_event, flags,
                                           start_event != nullptr || stop_event != nullptr ||
                                               flags != 0};
    return FP4Q_OK;
}

const char* fp4q_status_string(fp4q_status_t s) {
    switch (s) {
        case FP4Q_OK: return "ok";
        case FP4Q_ERR_INVALID: return "invalid argument";
        case FP4Q_ERR_UNSUPPORTED: return "unsupported";
        case FP4Q_ERR_ALIGNMENT: return "misaligned pointer or stride";
        case FP4Q_ERR_WORKSPACE: return "workspace too small";
        case FP4Q_ERR_HIP: return "HIP error";
    }
    return "unknown status";
}

fp4q_status_t fp4q_quantize(const void* x, fp4q_dtype_t x_dtype, int64_t rows, int64_t cols,
                            int64_t ld_x, int32_t block, fp4q_axis_t axis, fp4q_round_t round,
                            uint64_t seed, uint64_t rng_offset, uint8_t* codes, uint8_t* scales,
                            void* stream) {
    if (!x || !codes || !scales) return fail(FP4Q_ERR_INVALID, "quantize: null pointer");
    if (!valid_dtype(x_dtype)) return fail(FP4Q_ERR_INVALID, "quantize: bad x dtype %d", x_dtype);
    if (rows <= 0 || cols <= 0)
        return fail(FP4Q_ERR_INVALID, "quantize: rows=%lld cols=%lld", (long long)rows,
                    (long long)cols);
    if (ld_x < cols) return fail(FP4Q_ERR_INVALID, "quantize: ld_x < cols");
    if (!valid_block(block)) return fail(FP4Q_ERR_INVALID, "quantize: block %d", block);
    if (axis != FP4Q_BLOCK_ROW && axis != FP4Q_BLOCK_COL)
        return fail(FP4Q_ERR_INVALID, "quantize: bad axis");
    if (round != FP4Q_RNE && round != FP4Q_SR) return fail(FP4Q_ERR_INVALID, "quantize: bad round");
    if (axis == FP4Q_BLOCK_ROW && cols % block)
        return fail(FP4Q_ERR_INVALID, "quantize: cols %% block != 0 for ROW blocks");
    if (axis == FP4Q_BLOCK_COL && rows % block)
        return fail(FP4Q_ERR_INVALID, "quantize: rows %% block != 0 for COL blocks");
    if (rows > kMaxElems / ld_x) return fail(FP4Q_ERR_INVALID, "quantize: tensor too large");
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) ||
        (ld_x * esize(x_dtype)) % 16)
        return fail(FP4Q_ERR_ALIGNMENT, "quantize: pointers and row stride must be 16-byte aligned");
    hipError_t e;
    if (axis == FP4Q_BLOCK_ROW)
        e = fp4q::launch_quantize_row(x, x_dtype, rows, cols, ld_x, block, round == FP4Q_SR, seed,
                                      rng_offset, codes, scales, (hipStream_t)stream);
    else
        e = fp4q::launch_quantize_col(x, x_dtype, rows, cols, ld_x, block, round == FP4Q_SR, seed,
                                      rng_offset, codes, scales, (hipStream_t)stream);
    return hip_status(e, "quantize launch");
}

fp4q_status_t fp4q_channel_mask(const int32_t* idx, int32_t n, int64_t length, uint32_t* mask,
                                void* stream) {
    if (!mask || (n > 0 && !idx)) return fail(FP4Q_ERR_INVALID, "channel_mask: null pointer");
    if (n < 0 || length <= 0 || length >= ((int64_t)1 << 40))
        return fail(FP4Q_ERR_INVALID, "channel_mask: bad sizes");
    if (((uintptr_t)mask % 4) || (idx && ((uintptr_t)idx % 4)))
        return fail(FP4Q_ERR_ALIGNMENT, "channel_mask: pointers must be 4-byte aligned");
    return hip_status(fp4q::launch_channel_mask(idx, n, length, mask, (hipStream_t)stream),
                      "channel_mask launch");
}

fp4q_status_t fp4q_quantize_masked(const void* x, fp4q_dtype_t x_dtype, int64_t rows,
                                   int64_t cols, int64_t ld_x, int32_t block, fp4q_axis_t axis,
                                   fp4q_round_t round, uint64_t seed, uint64_t rng_offset,
                                   const uint32_t* zero_mask, uint8_t* codes, uint8_t* scales,
                                   void* stream) {
    if (!zero_mask) return fail(FP4Q_ERR_INVALID, "quantize_masked: null zero_mask");
    if ((uintptr_t)zero_mask % 4)
        return fail(FP4Q_ERR_ALIGNMENT, "quantize_masked: zero_mask must be 4-byte aligned");
    if (!x || !codes || !scales) return fail(FP4Q_ERR_INVALID, "quantize_masked: null pointer");
    if (!valid_dtype(x_dtype)) return fail(FP4Q_ERR_INVALID, "quantize_masked: bad x dtype");
    if (rows <= 0 || cols <= 0) return fail(FP4Q_ERR_INVALID, "quantize_masked: bad sizes");
    if (ld_x < cols) return fail(FP4Q_ERR_INVALID, "quantize_masked: ld_x < cols");
    if (!valid_block(block)) return fail(FP4Q_ERR_INVALID, "quantize_masked: block %d", block);
    if (axis != FP4Q_BLOCK_ROW && axis != FP4Q_BLOCK_COL)
        return fail(FP4Q_ERR_INVALID, "quantize_masked: bad axis");
    if (round != FP4Q_RNE && round != FP4Q_SR)
        return fail(FP4Q_ERR_INVALID, "quantize_masked: bad round");
    if (axis == FP4Q_BLOCK_ROW && cols % block)
        return fail(FP4Q_ERR_INVALID, "quantize_masked: cols %% block != 0 for ROW blocks");
    if (axis == FP4Q_BLOCK_COL && rows % block)
        return fail(FP4Q_ERR_INVALID, "quantize_masked: rows %% block != 0 for COL blocks");
    if (rows > kMaxElems / ld_x) return fail(FP4Q_ERR_INVALID, "quantize_masked: tensor too large");
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) ||
        (ld_x * esize(x_dtype)) % 16)
        return fail(FP4Q_ERR_ALIGNMENT,
                    "quantize_masked: pointers and row stride must be 16-byte aligned");
    hipError_t e;
    if (axis == FP4Q_BLOCK_ROW)
        e = fp4q::launch_quantize_row(x, x_dtype, rows, cols, ld_x, block, round == FP4Q_SR, seed,
                                      rng_offset, codes, scales, (hipStream_t)stream, zero_mask);
    else
        e = fp4q::launch_quantize_col(x, x_dtype, rows, cols, ld_x, block, round == FP4Q_SR, seed,
                                      rng_offset, codes, scales, (hipStream_t)stream, zero_mask);
    return hip_status(e, "quantize_masked launch");
}

fp4q_status_t fp4q_quantize_dual(const void* x, fp4q_dtype_t x_dtype, int64_t rows, int64_t cols,
                                 int64_t ld_x, int32_t block, fp4q_round_t round_row,
                                 uint64_t seed_row, fp4q_round_t round_col, uint64_t seed_col,
                                 uint64_t rng_offset, uint8_t* row_codes, uint8_t* row_scales,
                                 uint8_t* col_codes, uint8_t* col_scales, void* stream) {
    if (!x || !row_codes || !row_scales || !col_codes || !col_scales)
        return fail(FP4Q_ERR_INVALID, "quantize_dual: null pointer");
    if (!valid_dtype(x_dtype)) return fail(FP4Q_ERR_INVALID, "quantize_dual: bad x dtype %d", x_dtype);
    if (rows <= 0 || cols <= 0)
        return fail(FP4Q_ERR_INVALID, "quantize_dual: rows=%lld cols=%lld", (long long)rows,
                    (long long)cols);
    if (ld_x < cols) return fail(FP4Q_ERR_INVALID, "quantize_dual: ld_x < cols");
    if (!valid_block(block)) return fail(FP4Q_ERR_INVALID, "quantize_dual: block %d", block);
    if ((round_row != FP4Q_RNE && round_row != FP4Q_SR) ||
        (round_col != FP4Q_RNE && round_col != FP4Q_SR))
        return fail(FP4Q_ERR_INVALID, "quantize_dual: bad round");
    if (rows % block || cols % block)
        return fail(FP4Q_ERR_INVALID, "quantize_dual: rows and cols must be multiples of block");
    if (rows > kMaxElems / ld_x) return fail(FP4Q_ERR_INVALID, "quantize_dual: tensor too large");
    if (!aligned16(x) || !aligned16(row_codes) || !aligned16(row_scales) || !aligned16(col_codes) ||
        !aligned16(col_scales) || (ld_x * esize(x_dtype)) % 16)
        return fail(FP4Q_ERR_ALIGNMENT,
                    "quantize_dual: pointers and row stride must be 16-byte aligned");
    hipError_t e;
    if (x_dtype == FP4Q_BF16) {
        e = fp4q::launch_quantize_dual(x, rows, cols, ld_x, block, round_row == FP4Q_SR, seed_row,
                                       round_col == FP4Q_SR, seed_col, rng_offset, row_codes,
                                       row_scales, col_codes, col_scales, (hipStream_t)stream);
    } else {
        // fp32 input: the two passes run as separate launches
        e = fp4q::launch_quantize_row(x, x_dtype, rows, cols, ld_x, block, round_row == FP4Q_SR,
                                      seed_row, rng_offset, row_codes, row_scales,
                                      (hipStream_t)stream);
        if (e == hipSuccess)
            e = fp4q::launch_quantize_col(x, x_dtype, rows, cols, ld_x, block,
                                          round_col == FP4Q_SR, seed_col, rng_offset, col_codes,
                                          col_scales, (hipStream_t)stream);
    }
    return hip_status(e, "quantize_dual launch");
}

fp4q_status_t fp4q_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows,
                              int64_t k, int32_t block, void* y, fp4q_dtype_t y_dtype,
                              void* stream) {
    if (!codes || !scales || !y) return fail(FP4Q_ERR_INVALID, "dequantize: null pointer");
    if (!valid_dtype(y_dtype)) return fail(FP4Q_ERR_INVALID, "dequantize: bad y dtype");
    if (rows <= 0 || k <= 0) return fail(FP4Q_ERR_INVALID, "dequantize: bad sizes");
    if (!valid_block(block)) return fail(FP4Q_ERR_INVALID, "dequantize: block %d", block);
    if (k % block) return fail(FP4Q_ERR_INVALID, "dequantize: k %% block != 0");
    if (rows > kMaxElems / k) return fail(FP4Q_ERR_INVALID, "dequantize: tensor too large");
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(y))
        return fail(FP4Q_ERR_ALIGNMENT, "dequantize: pointers must be 16-byte aligned");
    return hip_status(fp4q::launch_dequantize(codes, scales, rows, k, block, y, y_dtype,
                                              (hipStream_t)stream),
                      "dequantize launch");
}

fp4q_status_t fp4q_grad_estimate(fp4q_grad_t mode, const void* x, fp4q_dtype_t x_dtype,
                                 const void* grad, fp4q_dtype_t g_dtype, int64_t rows,
                                 int64_t cols, int32_t block, fp4q_axis_t axis, float k,
                                 float clamp_max, void* out, fp4q_dtype_t out_dtype,
                                 void* stream) {
    if (mode != FP4Q_STE && mode != FP4Q_DGE) return fail(FP4Q_ERR_INVALID, "grad: bad mode");
    if (!grad || !out || (mode == FP4Q_DGE && !x))
        return fail(FP4Q_ERR_INVALID, "grad: null pointer");
    if (!valid_dtype(g_dtype) || !valid_dtype(out_dtype) ||
        (mode == FP4Q_DGE && !valid_dtype(x_dtype)))
        return fail(FP4Q_ERR_INVALID, "grad: bad dtype");
    if (rows <= 0 || cols <= 0) return fail(FP4Q_ERR_INVALID, "grad: bad sizes");
    if (rows > kMaxElems / cols) return fail(FP4Q_ERR_INVALID, "grad: tensor too large");
    if (!aligned16(grad) || !aligned16(out) || (x && !aligned16(x)))
        return fail(FP4Q_ERR_ALIGNMENT, "grad: pointers must be 16-byte aligned");
    if (mode == FP4Q_STE)
        return hip_status(fp4q::launch_ste(grad, g_dtype, rows * cols, out, out_dtype,
                                           (hipStream_t)stream),
                          "ste launch");
    if (!valid_block(block)) return fail(FP4Q_ERR_INVALID, "grad: block %d", block);
    if (axis != FP4Q_BLOCK_ROW && axis != FP4Q_BLOCK_COL)
        return fail(FP4Q_ERR_INVALID, "grad: bad axis");
    if (axis == FP4Q_BLOCK_ROW && cols % block)
        return fail(FP4Q_ERR_INVALID, "grad: cols %% block != 0 for ROW blocks");
    if (axis == FP4Q_BLOCK_COL && rows % block)
        return fail(FP4Q_ERR_INVALID, "grad: rows %% block != 0 for COL blocks");
    if (!(k >= 1.0f) || !(k < 1e30f)) return fail(FP4Q_ERR_INVALID, "grad: k must be >= 1");
    if (!(clamp_max > 0.0f)) return fail(FP4Q_ERR_INVALID, "grad: clamp_max must be > 0");
    return hip_status(fp4q::launch_dge(x, x_dtype, grad, g_dtype, rows, cols, block, axis, k,
                                       clamp_max, out, out_dtype, (hipStream_t)stream),
                      "dge launch");
}

fp4q_status_t fp4q_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                        const uint8_t* a_scales, const uint8_t* b_codes, const uint8_t* b_scales,
                        int32_t block, void* c, fp4q_dtype_t c_dtype, int64_t ld_c,
                        int32_t accumulate, void* stream) {
    if (!a_codes || !a_scales || !b_codes || !b_scales || !c)
        return fail(FP4Q_ERR_INVALID, "gemm: null pointer");
    if (M <= 0 || N <= 0 || K <= 0) return fail(FP4Q_ERR_INVALID, "gemm: bad sizes");
    if (!valid_dtype(c_dtype)) return fail(FP4Q_ERR_INVALID, "gemm: bad C dtype");
    if (!valid_block(block)) return fail(FP4Q_ERR_INVALID, "gemm: block %d", block);
    if (block != 32)
        return fail(FP4Q_ERR_UNSUPPORTED, "gemm: only block 32 (the MX hardware block)");
    if (K % 64) return fail(FP4Q_ERR_INVALID, "gemm: K %% 64 != 0");
    if (ld_c < N) return fail(FP4Q_ERR_INVALID, "gemm: ld_c < N");
    if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31) || K >= ((int64_t)1 << 31))
        return fail(FP4Q_ERR_INVALID, "gemm: dimension too large");
    if (K >= ((int64_t)1 << 24))
        return fail(FP4Q_ERR_UNSUPPORTED, "gemm: K must be below 2^24");
    if (accumulate != 0 && accumulate != 1) return fail(FP4Q_ERR_INVALID, "gemm: accumulate");
    if (accumulate && c_dtype != FP4Q_F32)
        return fail(FP4Q_ERR_UNSUPPORTED, "gemm: accumulate needs an fp32 C");
    if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) ||
        !aligned16(b_scales) || ((uintptr_t)c % (uintptr_t)esize(c_dtype)))
        return fail(FP4Q_ERR_ALIGNMENT,
                    "gemm: operand pointers must be 16-byte aligned, C element-aligned");
    return hip_status(fp4q::launch_gemm_fp4(M, N, K, a_codes, a_scales, b_codes, b_scales, c,
                                            c_dtype, ld_c, accumulate != 0, (hipStream_t)stream),
                      "gemm launch");
}

size_t fp4q_hcp_workspace_bytes(int64_t M, int64_t N, int32_t n_hot) {
    if (M <= 0 || N <= 0 || n_hot < 0) return 0;
    return fp4q::hcp_workspace_bytes(M, N, n_hot);
}

fp4q_status_t fp4q_hcp_residual_add(int64_t M, int64_t N, int64_t K, const void* x,
                                    const uint8_t* xq_codes, const uint8_t* xq_scales,
                                    const void* w, const uint8_t* wq_codes,
                                    const uint8_t* wq_scales, const int32_t* hot_idx,
                                    int32_t n_hot, float* y, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    if (M <= 0 || N <= 0 || K <= 0 || n_hot < 0) return fail(FP4Q_ERR_INVALID, "hcp: bad sizes");
    if (n_hot > K) return fail(FP4Q_ERR_INVALID, "hcp: n_hot > K");
    if (K % 32) return fail(FP4Q_ERR_INVALID, "hcp: K %% 32 != 0");
    if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31))
        return fail(FP4Q_ERR_INVALID, "hcp: dimension too large");
    if (n_hot > (1 << 20)) return fail(FP4Q_ERR_UNSUPPORTED, "hcp: n_hot above 2^20");
    if (n_hot == 0) return FP4Q_OK;
    if (!x || !xq_codes || !xq_scales || !w || !wq_codes || !wq_scales || !hot_idx || !y ||
        !workspace)
        return fail(FP4Q_ERR_INVALID, "hcp: null pointer");
    if (!aligned16(x) || !aligned16(xq_codes) || !aligned16(xq_scales) || !aligned16(w) ||
        !aligned16(wq_codes) || !aligned16(wq_scales) || !aligned16(hot_idx) || !aligned16(y) ||
        !aligned16(workspace))
        return fail(FP4Q_ERR_ALIGNMENT, "hcp: pointers must be 16-byte aligned");
    const size_t need = fp4q::hcp_workspace_bytes(M, N, n_hot);
    if (workspace_bytes < need)
        return fail(FP4Q_ERR_WORKSPACE, "hcp: workspace %zu < %zu bytes", workspace_bytes, need);
    return hip_status(fp4q::launch_hcp(M, N, K, x, xq_codes, xq_scales, w, wq_codes, wq_scales,
                                       hot_idx, n_hot, y, workspace, (hipStream_t)stream),
                      "hcp launch");
}

fp4q_status_t fp4q_hcp_residual_add_noalloc(int64_t M, int64_t N, int64_t K, const void* x,
                                            const uint8_t* xq_codes, const uint8_t* xq_scales,
                                            const void* w, const uint8_t* wq_codes,
                                            const uint8_t* wq_scales, const int32_t* hot_idx,
                                            int32_t n_hot, float* y, void* stream) {
    if (M <= 0 || N <= 0 || K <= 0 || n_hot < 0)
        return fail(FP4Q_ERR_INVALID, "hcp_noalloc: bad sizes");
    if (n_hot > K) return fail(FP4Q_ERR_INVALID, "hcp_noalloc: n_hot > K");
    if (K % 32) return fail(FP4Q_ERR_INVALID, "hcp_noalloc: K %% 32 != 0");
    if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31))
        return fail(FP4Q_ERR_INVALID, "hcp_noalloc: dimension too large");
    if (n_hot > (1 << 20)) return fail(FP4Q_ERR_UNSUPPORTED, "hcp_noalloc: n_hot above 2^20");
    if (n_hot == 0) return FP4Q_OK;
    if (!x || !xq_codes || !xq_scales || !w || !wq_codes || !wq_scales || !hot_idx || !y)
        return fail(FP4Q_ERR_INVALID, "hcp_noalloc: null pointer");
    if (!aligned16(x) || !aligned16(xq_codes) || !aligned16(xq_scales) || !aligned16(w) ||
        !aligned16(wq_codes) || !aligned16(wq_scales) || !aligned16(hot_idx) || !aligned16(y))
        return fail(FP4Q_ERR_ALIGNMENT, "hcp_noalloc: pointers must be 16-byte aligned");
    const size_t need = fp4q::hcp_workspace_bytes(M, N, n_hot);
    if (need > fp4q::kHcpStaticScratchBytes)
        return fail(FP4Q_ERR_WORKSPACE,
                    "hcp_noalloc: these sizes need %zu bytes of scratch, above the library's "
                    "static maximum of %zu (use fp4q_hcp_residual_add with a workspace)",
                    need, fp4q::kHcpStaticScratchBytes);
    void* ws = nullptr;
    fp4q_status_t st = hip_status(fp4q::hcp_static_scratch(&ws), "hcp_noalloc scratch address");
    if (st != FP4Q_OK) return st;
    return hip_status(fp4q::launch_hcp(M, N, K, x, xq_codes, xq_scales, w, wq_codes, wq_scales,
                                       hot_idx, n_hot, y, ws, (hipStream_t)stream),
                      "hcp_noalloc launch");
}

fp4q_status_t fp4q_gemm_dge(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                            const uint8_t* a_scales, const uint8_t* b_codes,
                            const uint8_t* b_scales, const void* x, fp4q_dtype_t x_dtype,
                            float k, float clamp_max, float* out, int64_t ld_out, void* stream) {
    if (!a_codes || !a_scales || !b_codes || !b_scales || !x || !out)
        return fail(FP4Q_ERR_INVALID, "gemm_dge: null pointer");
    if (M <= 0 || N <= 0 || K <= 0) return fail(FP4Q_ERR_INVALID, "gemm_dge: bad sizes");
    if (!valid_dtype(x_dtype)) return fail(FP4Q_ERR_INVALID, "gemm_dge: bad x dtype");
    if (x_dtype != FP4Q_BF16) return fail(FP4Q_ERR_UNSUPPORTED, "gemm_dge: x must be bf16");
    if (K % 64) return fail(FP4Q_ERR_INVALID, "gemm_dge: K %% 64 != 0");
    if (M % 32) return fail(FP4Q_ERR_INVALID, "gemm_dge: M %% 32 != 0 (column blocks of x)");
    if (ld_out < N) return fail(FP4Q_ERR_INVALID, "gemm_dge: ld_out < N");
    if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31))
        return fail(FP4Q_ERR_INVALID, "gemm_dge: dimension too large");
    if (M > kMaxElems / N) return fail(FP4Q_ERR_INVALID, "gemm_dge: tensor too large");
    if (K >= ((int64_t)1 << 24))
        return fail(FP4Q_ERR_UNSUPPORTED, "gemm_dge: K must be below 2^24");
    if (!(k >= 1.0f) || !(k < 1e30f)) return fail(FP4Q_ERR_INVALID, "gemm_dge: k must be >= 1");
    if (!(clamp_max > 0.0f)) return fail(FP4Q_ERR_INVALID, "gemm_dge: clamp_max must be > 0");
    if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) ||
        !aligned16(b_scales) || !aligned16(x) || ((uintptr_t)out % 4))
        return fail(FP4Q_ERR_ALIGNMENT,
                    "gemm_dge: operands and x must be 16-byte aligned, out 4-byte aligned");
    return hip_status(fp4q::launch_gemm_fp4_dge(M, N, K, a_codes, a_scales, b_codes, b_scales,
                                                (const uint16_t*)x, k, clamp_max, out, ld_out,
                                                (hipStream_t)stream),
                      "gemm_dge launch");
}

fp4q_status_t fp4q_gemm_quant(int64_t M, int64_t N, int64_t K, const uint8_t* a_codes,
                              const uint8_t* a_scales, const uint8_t* b_codes,
                              const uint8_t* b_scales, void* c, int64_t ld_c, uint8_t* y_codes,
                              uint8_t* y_scales, void* stream) {
    if (!a_codes || !a_scales || !b_codes || !b_scales || !y_codes || !y_scales)
        return fail(FP4Q_ERR_INVALID, "gemm_quant: null pointer");
    if (M <= 0 || N <= 0 || K <= 0) return fail(FP4Q_ERR_INVALID, "gemm_quant: bad sizes");
    if (K % 64) return fail(FP4Q_ERR_INVALID, "gemm_quant: K %% 64 != 0");
    if (N % 32) return fail(FP4Q_ERR_INVALID, "gemm_quant: N %% 32 != 0 (ROW blocks of C)");
    if (c && ld_c < N) return fail(FP4Q_ERR_INVALID, "gemm_quant: ld_c < N");
    if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31))
        return fail(FP4Q_ERR_INVALID, "gemm_quant: dimension too large");
    if (K >= ((int64_t)1 << 24))
        return fail(FP4Q_ERR_UNSUPPORTED, "gemm_quant: K must be below 2^24");
    if (!aligned16(a_codes) || !aligned16(a_scales) || !aligned16(b_codes) ||
        !aligned16(b_scales) || !aligned16(y_codes) || ((uintptr_t)c % 2))
        return fail(FP4Q_ERR_ALIGNMENT,
                    "gemm_quant: operands and codes 16-byte aligned, C element-aligned");
    return hip_status(fp4q::launch_gemm_fp4_quant(M, N, K, a_codes, a_scales, b_codes, b_scales,
                                                  (uint16_t*)c, ld_c, y_codes, y_scales,
                                                  (hipStream_t)stream),
                      "gemm_quant launch");
}

fp4q_status_t fp4q_gemm_hcp_split(int64_t M, int64_t N, int64_t K, const void* x,
                                  const uint8_t* xq_codes, const uint8_t* xq_scales,
                                  const void* w, const uint8_t* wq_codes,
                                  const uint8_t* wq_scales, const int32_t* hot_idx,
                                  int32_t n_hot, float* y, int64_t ld_y, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    if (M <= 0 || N <= 0 || K <= 0 || n_hot < 0)
        return fail(FP4Q_ERR_INVALID, "gemm_hcp_split: bad sizes");
    if (!xq_codes || !xq_scales || !wq_codes || !wq_scales || !y)
        return fail(FP4Q_ERR_INVALID, "gemm_hcp_split: null pointer");
    if (K % 64) return fail(FP4Q_ERR_INVALID, "gemm_hcp_split: K %% 64 != 0");
    if (ld_y < N) return fail(FP4Q_ERR_INVALID, "gemm_hcp_split: ld_y < N");
    if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31))
        return fail(FP4Q_ERR_INVALID, "gemm_hcp_split: dimension too large");
    if (K >= ((int64_t)1 << 24))
        return fail(FP4Q_ERR_UNSUPPORTED, "gemm_hcp_split: K must be below 2^24");
    if (n_hot > K) return fail(FP4Q_ERR_INVALID, "gemm_hcp_split: n_hot > K");
    if (n_hot > (1 << 20)) return fail(FP4Q_ERR_UNSUPPORTED, "gemm_hcp_split: n_hot above 2^20");
    if (!aligned16(xq_codes) || !aligned16(xq_scales) || !aligned16(wq_codes) ||
        !aligned16(wq_scales) || ((uintptr_t)y % 4))
        return fail(FP4Q_ERR_ALIGNMENT,
                    "gemm_hcp_split: operand pointers must be 16-byte aligned, y 4-byte aligned");
    if (n_hot > 0) {
        if (!x || !w || !hot_idx || !workspace)
            return fail(FP4Q_ERR_INVALID, "gemm_hcp_split: null pointer");
        if (!aligned16(x) || !aligned16(w) || !aligned16(hot_idx) || !aligned16(workspace))
            return fail(FP4Q_ERR_ALIGNMENT, "gemm_hcp_split: pointers must be 16-byte aligned");
        const size_t need = fp4q::hcp_workspace_bytes(M, N, n_hot);
        if (workspace_bytes < need)
            return fail(FP4Q_ERR_WORKSPACE, "gemm_hcp_split: workspace %zu < %zu bytes",
                        workspace_bytes, need);
    }
    return hip_status(fp4q::launch_gemm_hcp_split(M, N, K, x, xq_codes, xq_scales, w, wq_codes,
                                                  wq_scales, hot_idx, n_hot, y, ld_y, workspace,
                                                  (hipStream_t)stream),
                      "gemm_hcp_split launch");
}

fp4q_status_t fp4q_gemm_hcp(int64_t M, int64_t N, int64_t K, const void* x,
                            const uint8_t* xq_codes, const uint8_t* xq_scales, const void* w,
                            const uint8_t* wq_codes, const uint8_t* wq_scales,
                            const int32_t* hot_idx, int32_t n_hot, float* y, int64_t ld_y,
                            void* workspace, size_t workspace_bytes, void* stream) {
    if (M <= 0 || N <= 0 || K <= 0 || n_hot < 0)
        return fail(FP4Q_ERR_INVALID, "gemm_hcp: bad sizes");
    if (!xq_codes || !xq_scales || !wq_codes || !wq_scales || !y)
        return fail(FP4Q_ERR_INVALID, "gemm_hcp: null pointer");
    if (K % 64) return fail(FP4Q_ERR_INVALID, "gemm_hcp: K %% 64 != 0");
    if (ld_y < N) return fail(FP4Q_ERR_INVALID, "gemm_hcp: ld_y < N");
    if (M >= ((int64_t)1 << 31) || N >= ((int64_t)1 << 31))
        return fail(FP4Q_ERR_INVALID, "gemm_hcp: dimension too large");
    if (K >= ((int64_t)1 << 24))
        return fail(FP4Q_ERR_UNSUPPORTED, "gemm_hcp: K must be below 2^24");
    if (n_hot > K) return fail(FP4Q_ERR_INVALID, "gemm_hcp: n_hot > K");
    if (n_hot > (1 << 20)) return fail(FP4Q_ERR_UNSUPPORTED, "gemm_hcp: n_hot above 2^20");
    if (!aligned16(xq_codes) || !aligned16(xq_scales) || !aligned16(wq_codes) ||
        !aligned16(wq_scales) || ((uintptr_t)y % 4))
        return fail(FP4Q_ERR_ALIGNMENT,
                    "gemm_hcp: operand pointers must be 16-byte aligned, y 4-byte aligned");
    if (n_hot > 0) {
        if (!x || !w || !hot_idx || !workspace)
            return fail(FP4Q_ERR_INVALID, "gemm_hcp: null pointer");
        if (!aligned16(x) || !aligned16(w) || !aligned16(hot_idx) || !aligned16(workspace))
            return fail(FP4Q_ERR_ALIGNMENT, "gemm_hcp: pointers must be 16-byte aligned");
        const size_t need = fp4q::hcp_workspace_bytes(M, N, n_hot);
        if (workspace_bytes < need)
            return fail(FP4Q_ERR_WORKSPACE, "gemm_hcp: workspace %zu < %zu bytes",
                        workspace_bytes, need);
    }
    return hip_status(fp4q::launch_gemm_hcp(M, N, K, x, xq_codes, xq_scales, w, wq_codes,
                                            wq_scales, hot_idx, n_hot, y, ld_y, workspace,
                                            (hipStream_t)stream),
                      "gemm_hcp launch");
}

size_t fp4q_hot_channels_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return fp4q::hot_channels_workspace_bytes(rows, cols);
}

fp4q_status_t fp4q_hot_channels(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                int32_t n_hot, int32_t* hot_idx, float* err, void* workspace,
                                size_t workspace_bytes, void* stream) {
    if (rows <= 0 || cols <= 0 || n_hot < 0)
        return fail(FP4Q_ERR_INVALID, "hot_channels: rows=%lld cols=%lld n_hot=%d",
                    (long long)rows, (long long)cols, (int)n_hot);
    if (!x || !workspace || (n_hot > 0 && !hot_idx))
        return fail(FP4Q_ERR_INVALID, "hot_channels: null pointer");
    if (cols % 32) return fail(FP4Q_ERR_INVALID, "hot_channels: cols %% 32 != 0");
    if (ld_x < cols || ld_x % 8)
        return fail(FP4Q_ERR_INVALID, "hot_channels: ld_x must be >= cols and a multiple of 8");
    if (n_hot > cols) return fail(FP4Q_ERR_INVALID, "hot_channels: n_hot > cols");
    if (cols > fp4q::hot_channels_max_cols())
        return fail(FP4Q_ERR_UNSUPPORTED, "hot_channels: cols above %lld",
                    (long long)fp4q::hot_channels_max_cols());
    if (rows > kMaxElems / ld_x) return fail(FP4Q_ERR_INVALID, "hot_channels: tensor too large");
    if (!aligned16(x) || !aligned16(workspace) || ((uintptr_t)hot_idx % 4) ||
        ((uintptr_t)err % 4))
        return fail(FP4Q_ERR_ALIGNMENT,
                    "hot_channels: x and workspace 16-byte aligned, hot_idx and err 4-byte");
    const size_t need = fp4q::hot_channels_workspace_bytes(rows, cols);
    if (workspace_bytes < need)
        return fail(FP4Q_ERR_WORKSPACE, "hot_channels: workspace %zu < %zu bytes",
                    workspace_bytes, need);
    return hip_status(fp4q::launch_hot_channels((const uint16_t*)x, rows, cols, ld_x, n_hot,
                                                workspace, hot_idx, err, (hipStream_t)stream),
                      "hot_channels launch");
}

fp4q_status_t fp4q_quantize_2d_tile(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                    int32_t tile, fp4q_round_t round, uint64_t seed,
                                    uint64_t rng_offset, uint8_t* row_codes, uint8_t* row_scales,
                                    uint8_t* col_codes, uint8_t* col_scales, void* stream) {
    if (!x || !row_codes || !row_scales || !col_codes || !col_scales)
        return fail(FP4Q_ERR_INVALID, "quantize_2d: null pointer");
    if (tile != 16 && tile != 32) return fail(FP4Q_ERR_INVALID, "quantize_2d: tile must be 16 or 32");
    if (rows <= 0 || cols <= 0)
        return fail(FP4Q_ERR_INVALID, "quantize_2d: rows=%lld cols=%lld", (long long)rows,
                    (long long)cols);
    if (rows % 32 || cols % 32)
        return fail(FP4Q_ERR_INVALID, "quantize_2d: rows and cols must be multiples of 32");
    if (ld_x < cols) return fail(FP4Q_ERR_INVALID, "quantize_2d: ld_x < cols");
    if (round != FP4Q_RNE && round != FP4Q_SR)
        return fail(FP4Q_ERR_INVALID, "quantize_2d: bad round");
    if (rows > kMaxElems / ld_x) return fail(FP4Q_ERR_INVALID, "quantize_2d: tensor too large");
    if (!aligned16(x) || !aligned16(row_codes) || !aligned16(row_scales) ||
        !aligned16(col_codes) || !aligned16(col_scales) || ld_x % 8)
        return fail(FP4Q_ERR_ALIGNMENT,
                    "quantize_2d: pointers and the row stride must be 16-byte aligned");
    return hip_status(fp4q::launch_quantize_2d(x, rows, cols, ld_x, tile, round == FP4Q_SR, seed,
                                               rng_offset, row_codes, row_scales, col_codes,
                                               col_scales, (hipStream_t)stream),
                      "quantize_2d launch");
}

fp4q_status_t fp4q_quantize_2d(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                               fp4q_round_t round, uint64_t seed, uint64_t rng_offset,
                               uint8_t* row_codes, uint8_t* row_scales, uint8_t* col_codes,
                               uint8_t* col_scales, void* stream) {
    return fp4q_quantize_2d_tile(x, rows, cols, ld_x, 32, round, seed, rng_offset, row_codes,
                                 row_scales, col_codes, col_scales, stream);
}

fp4q_status_t fp4q_quantize_rht(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                fp4q_axis_t axis, const uint32_t* signs, fp4q_round_t round,
                                uint64_t seed, uint64_t rng_offset, uint8_t* codes,
                                uint8_t* scales, void* stream) {
    if (!x || !signs || !codes || !scales)
        return fail(FP4Q_ERR_INVALID, "quantize_rht: null pointer");
    if (rows <= 0 || cols <= 0)
        return fail(FP4Q_ERR_INVALID, "quantize_rht: rows=%lld cols=%lld", (long long)rows,
                    (long long)cols);
    if (axis != FP4Q_BLOCK_ROW && axis != FP4Q_BLOCK_COL)
        return fail(FP4Q_ERR_INVALID, "quantize_rht: bad axis");
    if (round != FP4Q_RNE && round != FP4Q_SR)
        return fail(FP4Q_ERR_INVALID, "quantize_rht: bad round");
    if (axis == FP4Q_BLOCK_ROW && cols % 32)
        return fail(FP4Q_ERR_INVALID, "quantize_rht: cols %% 32 != 0 for ROW groups");
    if (axis == FP4Q_BLOCK_COL && (rows % 32 || cols % 2))
        return fail(FP4Q_ERR_INVALID, "quantize_rht: COL groups need rows %% 32 == 0, even cols");
    if (ld_x < cols) return fail(FP4Q_ERR_INVALID, "quantize_rht: ld_x < cols");
    if (rows > kMaxElems / ld_x) return fail(FP4Q_ERR_INVALID, "quantize_rht: tensor too large");
    if (axis == FP4Q_BLOCK_COL && rows / 32 > 65535)
        return fail(FP4Q_ERR_UNSUPPORTED, "quantize_rht: too many rows");
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || ((uintptr_t)signs % 4) ||
        ld_x % 8)
        return fail(FP4Q_ERR_ALIGNMENT,
                    "quantize_rht: x, codes, scales and the row stride 16-byte aligned, signs 4");
    return hip_status(fp4q::launch_quantize_rht(x, rows, cols, ld_x, axis == FP4Q_BLOCK_COL, signs,
                                                round == FP4Q_SR, seed, rng_offset, codes, scales,
                                                (hipStream_t)stream),
                      "quantize_rht launch");
}

static bool occ_rank(int64_t rows, int64_t cols, double quantile, int64_t* j) {
    if (rows <= 0 || cols <= 0 || !(quantile > 0.0 && quantile <= 1.0)) return false;
    const int64_t n = rows * cols;
    int64_t jj = (int64_t)ceil(quantile * (double)n);
    if (jj < 1) jj = 1;
    if (jj > n) jj = n;
    *j = jj;
    return true;
}

int64_t fp4q_occ_max_nnz(int64_t rows, int64_t cols, double quantile) {
    int64_t j;
    if (rows > ((int64_t)1 << 32) || cols > ((int64_t)1 << 32) || !occ_rank(rows, cols, quantile, &j))
        return -1;
    return rows * cols - j;
}

size_t fp4q_occ_workspace_bytes(int64_t rows, int64_t cols) {
    if (rows <= 0 || cols <= 0) return 0;
    return fp4q::occ_workspace_bytes(rows, cols);
}

fp4q_status_t fp4q_occ_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld_x,
                                double quantile, fp4q_round_t round, uint64_t seed,
                                uint64_t rng_offset, uint8_t* codes, uint8_t* scales,
                                int64_t* row_ptr, int32_t* col_idx, float* vals, int64_t nnz_cap,
                                uint16_t* threshold, void* workspace, size_t workspace_bytes,
                                void* stream) {
    if (!x || !codes || !scales || !row_ptr || !workspace)
        return fail(FP4Q_ERR_INVALID, "occ_quantize: null pointer");
    if (rows <= 0 || cols <= 0 || cols % 32)
        return fail(FP4Q_ERR_INVALID, "occ_quantize: rows > 0 and cols a positive multiple of 32");
    if (rows * cols >= ((int64_t)1 << 32))
        return fail(FP4Q_ERR_UNSUPPORTED, "occ_quantize: tensors of 2^32 elements or more");
    int64_t j;
    if (!occ_rank(rows, cols, quantile, &j))
        return fail(FP4Q_ERR_INVALID, "occ_quantize: quantile must lie in (0, 1]");
    if (round != FP4Q_RNE && round != FP4Q_SR) return fail(FP4Q_ERR_INVALID, "occ_quantize: bad round");
    if (ld_x < cols) return fail(FP4Q_ERR_INVALID, "occ_quantize: ld_x < cols");
    if (rows > kMaxElems / ld_x) return fail(FP4Q_ERR_INVALID, "occ_quantize: tensor too large");
    const int64_t bound = rows * cols - j;
    if (nnz_cap < bound)
        return fail(FP4Q_ERR_INVALID, "occ_quantize: nnz_cap %lld < %lld (fp4q_occ_max_nnz)",
                    (long long)nnz_cap, (long long)bound);
    if (bound > 0 && (!col_idx || !vals))
        return fail(FP4Q_ERR_INVALID, "occ_quantize: null residual arrays");
    if (!aligned16(x) || !aligned16(codes) || !aligned16(scales) || !aligned16(workspace) ||
        ld_x % 8 || ((uintptr_t)row_ptr % 8) || ((uintptr_t)col_idx % 4) || ((uintptr_t)vals % 4))
        return fail(FP4Q_ERR_ALIGNMENT, "occ_quantize: misaligned pointer or row stride");
    const size_t need = fp4q::occ_workspace_bytes(rows, cols);
    if (workspace_bytes < need)
        return fail(FP4Q_ERR_WORKSPACE, "occ_quantize: workspace %zu < %zu bytes", workspace_bytes,
                    need);
    int dev = 0, cus = 256;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
        return fail(FP4Q_ERR_HIP, "occ_quantize: device query failed");
    return hip_status(fp4q::launch_occ_quantize(x, rows, cols, ld_x, (uint64_t)j, round == FP4Q_SR,
                                                seed, rng_offset, codes, scales, row_ptr, col_idx,
                                                vals, threshold, workspace, cus,
                                                (hipStream_t)stream),
                      "occ_quantize launch");
}

fp4q_status_t fp4q_occ_spmm(int64_t M, int64_t N, int64_t K, const int64_t* row_ptr,
                            const int32_t* col_idx, const float* vals, const void* w,
                            int64_t ld_w, float* y, int64_t ld_y, void* stream) {
    if (M <= 0 || N <= 0 || K <= 0) return fail(FP4Q_ERR_INVALID, "occ_spmm: bad sizes");
    if (!row_ptr || !w || !y) return fail(FP4Q_ERR_INVALID, "occ_spmm: null pointer");
    if (N % 8) return fail(FP4Q_ERR_INVALID, "occ_spmm: N %% 8 != 0");
    if (ld_w < N || ld_y < N) return fail(FP4Q_ERR_INVALID, "occ_spmm: ld_w or ld_y < N");
    if (M > 2147483647LL || N / 2048 >= 65535)
        return fail(FP4Q_ERR_UNSUPPORTED, "occ_spmm: M or N too large");
    if (!aligned16(w) || !aligned16(y) || ld_w % 8 || ld_y % 4 || ((uintptr_t)row_ptr % 8) ||
        ((uintptr_t)col_idx % 4) || ((uintptr_t)vals % 4))
        return fail(FP4Q_ERR_ALIGNMENT, "occ_spmm: misaligned pointer or row stride");
    return hip_status(fp4q::launch_occ_spmm(M, N, row_ptr, col_idx, vals, w, ld_w, y, ld_y,
                                            (hipStream_t)stream),
                      "occ_spmm launch");
}

}  // extern "C"
