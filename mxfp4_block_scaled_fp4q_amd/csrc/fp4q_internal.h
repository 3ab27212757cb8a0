// Internal launcher interface between the C-ABI layer (fp4q_api.hip) and the
// kernel translation units.  Launchers assume validated arguments.
#pragma once
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

// Options for the next kernel this thread launches through the library
// (fp4q_set_next_launch): events recorded by that kernel's own dispatch, and
// kAnyOrder, which lets the kernel start before earlier work in its stream
// has finished.  The launch that takes them clears them.
constexpr uint32_t kAnyOrder = 1;
struct NextLaunch {
    hipEvent_t start, stop;
    uint32_t flags;
    bool pending;
};
extern thread_local NextLaunch g_next_launch;

// Every kernel launch of the library: plain, or, with options pending, through
// hipExtLaunchKernel (events at the dispatch; any-order launches carry no
// barrier behind the stream's earlier packets).
#define FP4Q_LAUNCH(KERNEL, GRID, BLOCK, LDS, STREAM, ...)                                \
    do {                                                                                \
        if (::fp4q::g_next_launch.pending) {                                            \
            const ::fp4q::NextLaunch nl_ = ::fp4q::g_next_launch;                       \
            ::fp4q::g_next_launch = ::fp4q::NextLaunch{nullptr, nullptr, 0u, false};    \
            hipExtLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, nl_.start, nl_.stop,  \
                                  (nl_.flags & ::fp4q::kAnyOrder) ? hipExtAnyOrderLaunch : 0u, \
                                  __VA_ARGS__);                                         \
        } else {                                                                        \
            hipLaunchKernelGGL(KERNEL, GRID, BLOCK, LDS, STREAM, __VA_ARGS__);          \
        }                                                                               \
    } while (0)

// n / d for n < 2^31 with a precomputed multiplier (Granlund & Montgomery,
// "Division by invariant integers using multiplication", PLDI'94, round-up
// variant): q = (umulhi(n, mul) + n) >> shift.
struct FastDiv {
    uint32_t d, mul, shift;
};
inline FastDiv make_fastdiv(uint32_t d) {
    FastDiv f;
    f.d = d;
    uint32_t l = 0;
    while ((1ull << l) < d) ++l;
    f.shift = l;
    f.mul = (uint32_t)(((1ull << 32) * ((1ull << l) - d)) / d + 1);
    return f;
}
__device__ __forceinline__ uint32_t fastdiv(uint32_t n, FastDiv f) {
    return (__umulhi(n, f.mul) + n) >> f.shift;
}

enum DType { F32 = 0, BF16 = 1 };

// zmask (optional): one bit per position along the block axis (ROW: columns,
// COL: rows); set positions are quantised as zeros.
hipError_t launch_quantize_row(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                               int block, bool sr, uint64_t seed, uint64_t off, uint8_t* codes,
                               uint8_t* scales, hipStream_t s, const uint32_t* zmask = nullptr);
hipError_t launch_quantize_col(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                               int block, bool sr, uint64_t seed, uint64_t off, uint8_t* codes,
                               uint8_t* scales, hipStream_t s, const uint32_t* zmask = nullptr);
// mask[0 .. ceil(length/32)) = bit i set for every i in idx[0 .. n) (0 <= i < length).
hipError_t launch_channel_mask(const int32_t* idx, int32_t n, int64_t length, uint32_t* mask,
                               hipStream_t s);
hipError_t launch_quantize_dual(const void* x, int64_t rows, int64_t cols, int64_t ld, int block,
                                bool sr_row, uint64_t seed_row, bool sr_col, uint64_t seed_col,
                                uint64_t off, uint8_t* codes_r, uint8_t* scales_r,
                                uint8_t* codes_c, uint8_t* scales_c, hipStream_t s);
hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                             int block, void* y, int ydtype, hipStream_t s);
hipError_t launch_ste(const void* g, int gdtype, int64_t n, void* out, int odtype, hipStream_t s);
hipError_t launch_dge(const void* x, int xdtype, const void* g, int gdtype, int64_t rows,
                      int64_t cols, int block, int axis, float k, float clamp_max, void* out,
                      int odtype, hipStream_t s);
hipError_t launch_gemm_fp4(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                           const uint8_t* as, const uint8_t* bc, const uint8_t* bs, void* c,
                           int cdtype, int64_t ldc, bool accumulate, hipStream_t s);
// C[M,N] (fp32, row stride ldc) += A B^T for bf16 A [M,K], B [N,K] (K % 32 == 0),
// on the FP4 GEMM's pipeline with bf16 MFMAs.
hipError_t launch_gemm_bf16_accum(int64_t M, int64_t N, int64_t K, const uint16_t* a,
                                  const uint16_t* b, float* c, int64_t ldc, hipStream_t s);
// C[M,N] (fp32, row stride ldc) = A B^T over FP4 operands (as launch_gemm_fp4)
// plus ha hb^T over kp-deep bf16 operands (kp % 32 == 0), in one kernel.
hipError_t launch_gemm_fp4_hot(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                               const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                               const uint16_t* ha, const uint16_t* hb, int64_t kp, float* c,
                               int64_t ldc, hipStream_t s);
// C[M,N] (fp32, row stride ldc) = (A B^T) * DGE'(x), x bf16 [M, N] dense with
// column blocks of 32 rows (M % 32 == 0, K % 128 == 0).
hipError_t launch_gemm_fp4_dge(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                               const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                               const uint16_t* x, float k, float clamp_max, float* c,
                               int64_t ldc, hipStream_t s);
// C[M,N] = A B^T rounded to bf16 (stored if c is not null) and that bf16 C
// quantised with ROW blocks of 32, nearest-even, into qc, qs (N % 32 == 0).
hipError_t launch_gemm_fp4_quant(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                                 const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                                 uint16_t* c, int64_t ldc, uint8_t* qc, uint8_t* qs,
                                 hipStream_t s);
size_t hcp_workspace_bytes(int64_t M, int64_t N, int32_t n_hot);
// Size of the library-owned scratch array fp4q_hcp_residual_add_noalloc uses
// instead of a caller workspace, and the device address of the current
// device's copy (taken once per device).
constexpr size_t kHcpStaticScratchBytes = (size_t)64 << 20;
constexpr int kMaxDevices = 64;
hipError_t hcp_static_scratch(void** out);
// Split reading: Y = Xq' Wq' + X_H W_H (Xq', Wq' quantised with H zeroed).
hipError_t launch_gemm_hcp_split(int64_t M, int64_t N, int64_t K, const void* x,
                                 const uint8_t* xqc, const uint8_t* xqs, const void* w,
                                 const uint8_t* wqc, const uint8_t* wqs, const int32_t* hot,
                                 int32_t n_hot, float* y, int64_t ldy, void* ws, hipStream_t s);
hipError_t launch_hcp(int64_t M, int64_t N, int64_t K, const void* x, const uint8_t* xqc,
                      const uint8_t* xqs, const void* w, const uint8_t* wqc, const uint8_t* wqs,
                      const int32_t* hot, int32_t n_hot, float* y, void* ws, hipStream_t s);
hipError_t launch_gemm_hcp(int64_t M, int64_t N, int64_t K, const void* x, const uint8_t* xqc,
                           const uint8_t* xqs, const void* w, const uint8_t* wqc,
                           const uint8_t* wqs, const int32_t* hot, int32_t n_hot, float* y,
                           int64_t ldy, void* ws, hipStream_t s);
// Hot-channel choice: per-column ROW block-32 RNE quantisation error of the
// bf16 X [rows, cols] and the n_hot columns of largest error, ascending.
size_t hot_channels_workspace_bytes(int64_t rows, int64_t cols);
int64_t hot_channels_max_cols();
hipError_t launch_hot_channels(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                               int32_t n_hot, void* ws, int32_t* hot, float* err_out,
                               hipStream_t s);
// 2D (32 x 32 square) block scaling of a bf16 [rows, cols]: the same codes
// in the ROW and the COL layout.
hipError_t launch_quantize_2d(const void* x, int64_t rows, int64_t cols, int64_t ld, int tile,
                              bool sr, uint64_t seed, uint64_t off, uint8_t* codes_r,
                              uint8_t* scales_r, uint8_t* codes_c, uint8_t* scales_c,
                              hipStream_t s);
// Block-32 quantisation of c * H32 * D * x along the block axis (ROW: along
// columns; COL: along rows, K-major output), D from the sign mask.
hipError_t launch_quantize_rht(const void* x, int64_t rows, int64_t cols, int64_t ld, bool col,
                               const uint32_t* signs, bool sr, uint64_t seed, uint64_t off,
                               uint8_t* codes, uint8_t* scales, hipStream_t s);
// Outlier clamping and compensation: threshold (the j-th smallest |x|),
// clamp + ROW block-32 quantisation, residual CSR; and the residual's
// product with a bf16 weight added into an fp32 output.
size_t occ_workspace_bytes(int64_t rows, int64_t cols);
hipError_t launch_occ_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, uint64_t j,
                               bool sr, uint64_t seed, uint64_t off, uint8_t* codes,
                               uint8_t* scales, int64_t* row_ptr, int32_t* col_idx, float* vals,
                               uint16_t* t_out, void* ws, int n_cus, hipStream_t s);
hipError_t launch_occ_spmm(int64_t M, int64_t N, const int64_t* row_ptr, const int32_t* col_idx,
                           const float* vals, const void* w, int64_t ldw, float* y, int64_t ldy,
                           hipStream_t s);

}  // namespace fp4q
