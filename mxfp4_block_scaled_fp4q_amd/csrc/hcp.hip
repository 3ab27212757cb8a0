// Hot-channel compensation, dual-kernel mode.
//
// The outlier-dynamics page (sec. 3.1) decomposes the quantised product as
// W^T X + (first-order terms W^T dX + dW^T X) + (second-order term dW^T dX)
// and offers a "D" mode in which the base GEMM and a residual GEMM over the
// hot channels run as separate kernels and are added; its sec. 3.2 sketch
// accumulates, per hot channel c, W[:,c] X[c,:] minus the quantised
// operands' product.  Here, for the hot set H:
//
//   Y[i, j] += sum_{c in H} ( X[i,c] W[c,j] - Xq[i,c] Wq[c,j] )
//
// which swaps, on H only, the FP4 operands' product for the bf16 operands'
// product (every error term of both operands on those channels).  It runs as
// one bf16 GEMM of depth K' = 2|H| (padded to 32):
//   A' = [X_H | Xq_H]    [M, K']   (gathered, dequantised)
//   B' = [W_H ; -Wq_H]^T [N, K']   (gathered, K-major)
// with fp32 accumulation, added into the fp32 Y in the epilogue.  The hot
// indices are a device array prepared once by the caller (the page's advice
// to precompute and cache them, sec. 3.2).  All dequantised values are exact
// in bf16 and every bf16 x bf16 product is exact in fp32.
//
// Single-kernel ("S") mode of the same section: the FP4 GEMM kernel runs its
// FP4 K loop over all K and then a bf16 K loop over the same A', B' into the
// same fp32 accumulators, so Y = Xq Wq + residual is written once and the
// fp32 read-modify-write of Y disappears.
//
// Split reading (the alternative the outlier-dynamics page's wording
// allows): the hot channels are taken out of the quantised product -- X's
// hot columns and W's hot rows are zeroed before quantisation (the
// quantisers' zero mask) -- and added back in bf16:
//   Y = Xq' Wq' + X_H W_H,  one kernel, K' = |H| padded to 32.
//
// Kernels:
//  * hcp_gather_x_rows: a workgroup stages a few whole rows of X (and of its
//    codes and scales) in LDS with coalesced 16-byte loads, then each lane
//    forms 8 consecutive K' slots of a row of A' from LDS.  The hot columns
//    are scattered over each row, so gathering them straight from HBM costs
//    one address per element (the load path, not HBM, was the limit); a row
//    read whole costs a few full-line loads.
//  * hcp_gather_x: one lane = 8 consecutive K' slots of one row of A', read
//    straight from global memory (rows too long to stage in LDS).
//  * hcp_gather_w_rows: a workgroup forms 4 rows of B' from LDS-staged
//    pieces (the hot rows' values at those 4 columns, and Wq's 4 K-major code
//    and scale rows read whole).
//  * hcp_gather_w: one lane = one column j and 8 consecutive K' slots; lanes
//    of a wave take consecutive j, so the reads of W's hot rows coalesce
//    (used where the staged pieces do not fit in LDS).
//  * the residual GEMM runs on the FP4 GEMM's kernel instantiated for bf16
//    operands (v_mfma_f32_32x32x16_bf16: lane l supplies row l % 32, K
//    elements [8 (l / 32), 8 (l / 32) + 8) -- the same 16 bytes per lane as
//    an FP4 fragment), adding into the fp32 Y in its epilogue.
#include <algorithm>

#include <mutex>

#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

static constexpr int kThreads = 256;
// rows of B' per workgroup of the row-staged W gather: 4 (about 18 KB of LDS
// at the 13B shape, 8 workgroups per compute unit) rather than 8 (33 KB, 4
// per unit): 51 -> 44 us in a same-box A/B
static constexpr int kGatherWRows = 4;

__device__ __forceinline__ float deq_nibble(const uint8_t* codes_row, const uint8_t* scales_row,
                                            int c) {
    const uint32_t byte = codes_row[c >> 1];
    const uint32_t code = (c & 1) ? (byte >> 4) : (byte & 0xFu);
    const uint32_t sb = scales_row[c >> 5];
    // E2M1 magnitude from the code bits: e = code[2:1], m = code[0]
    const uint32_t e = (code >> 1) & 3u, m = code & 1u;
    const float mag = e == 0 ? 0.5f * (float)m : (float)(2u + m) * as_f32((125u + e) << 23);
    const float v = (code & 8u) ? -mag : mag;
    if (sb == 0xFFu) return __builtin_nanf("");
    return v * e8m0_scale_f32(sb);
}

static size_t round_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

static int64_t padded_k(int32_t n_hot) { return (int64_t)round_up((size_t)(2 * n_hot), 32); }
// split reading: the hot channels alone, unpaired with their quantised copies
static int64_t padded_k_split(int32_t n_hot) { return (int64_t)round_up((size_t)n_hot, 32); }

size_t hcp_workspace_bytes(int64_t M, int64_t N, int32_t n_hot) {
    if (n_hot <= 0) return 0;
    const int64_t kp = padded_k(n_hot);
    return round_up((size_t)(M * kp * 2), 256) + round_up((size_t)(N * kp * 2), 256);
}

__global__ __launch_bounds__(kThreads) void hcp_gather_x(const uint16_t* __restrict__ x,
                                                         const uint8_t* __restrict__ xqc,
                                                         const uint8_t* __restrict__ xqs,
                                                         const int32_t* __restrict__ hot,
                                                         int n_hot, int64_t M, int64_t K,
                                                         int64_t kp, uint16_t* __restrict__ a,
                                                         int with_q) {
    const int64_t chunks_per_row = kp / 8;
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= M * chunks_per_row) return;
    const int64_t i = t / chunks_per_row;
    const int h0 = (int)(t - i * chunks_per_row) * 8;
    uint32_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int h = h0 + q;
        uint32_t bits = 0;
        if (h < n_hot) {
            bits = x[i * K + hot[h]];
        } else if (with_q && h < 2 * n_hot) {
            const int c = hot[h - n_hot];
            bits = f32_to_bf16_bits(deq_nibble(xqc + i * (K / 2), xqs + i * (K / 32), c));
        }
        v[q] = bits;
    }
    uint4 o;
    o.x = v[0] | (v[1] << 16);
    o.y = v[2] | (v[3] << 16);
    o.z = v[4] | (v[5] << 16);
    o.w = v[6] | (v[7] << 16);
    *(uint4*)(a + i * kp + h0) = o;
}

// LDS table of the column each of the kp slots of a gathered row takes:
// slot h < n_hot the hot column hot[h], slot n_hot + h (with_q) the same
// column's quantised copy, -1 (zero) for the padding and for an index outside
// [0, K) (a broken caller precondition).  The caller synchronises.
__device__ __forceinline__ void fill_slot_columns(int32_t* hs, const int32_t* __restrict__ hot,
                                                  int n_hot, int64_t kp, int with_q, int64_t K) {
    for (int h = threadIdx.x; h < kp; h += kThreads) {
        int src = h < n_hot ? h : (with_q && h < 2 * n_hot ? h - n_hot : -1);
        int c = src >= 0 ? hot[src] : -1;
        hs[h] = (c >= 0 && c < K) ? c : -1;
    }
}

// Row-staged gather: dynamic LDS holds the slot -> column table (kp int32),
// then RPW rows of row_bytes each: K bf16 of X, and with_q also K/2 code
// bytes and K/32 scale bytes.  K % 32 == 0, so the X and code
// rows are whole 16-byte words (the scale bytes are copied one by one).  A
// hot index outside [0, K) (a broken caller precondition) reads as zero.
__global__ __launch_bounds__(kThreads) void hcp_gather_x_rows(
    const uint16_t* __restrict__ x, const uint8_t* __restrict__ xqc,
    const uint8_t* __restrict__ xqs, const int32_t* __restrict__ hot, int n_hot, int64_t M,
    int64_t K, int64_t kp, uint16_t* __restrict__ a, int with_q, int rpw, int hot_bytes,
    int row_bytes) {
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int32_t* hs = (int32_t*)smem;  // slot -> column of X (-1: zero), kp entries
    const int tid = threadIdx.x;
    const int64_t i0 = (int64_t)blockIdx.x * rpw;
    fill_slot_columns(hs, hot, n_hot, kp, with_q, K);
    const int xw = (int)(K * 2 / 16), cw = (int)(K / 2 / 16), sw = (int)(K / 32);
    for (int r = 0; r < rpw; ++r) {
        const int64_t i = i0 + r;
        if (i >= M) break;
        uint8_t* row = smem + hot_bytes + r * row_bytes;
        const uint4* xs = (const uint4*)(x + i * K);
        for (int c = tid; c < xw; c += kThreads) ((uint4*)row)[c] = xs[c];
        if (with_q) {
            const uint4* cs = (const uint4*)(xqc + i * (K / 2));
            for (int c = tid; c < cw; c += kThreads) ((uint4*)(row + K * 2))[c] = cs[c];
            const uint8_t* ss = xqs + i * (K / 32);
            for (int c = tid; c < sw; c += kThreads) row[K * 2 + K / 2 + c] = ss[c];
        }
    }
    __syncthreads();
    const int cpr = (int)(kp / 8);
    for (int t = tid; t < rpw * cpr; t += kThreads) {
        const int r = t / cpr;
        const int64_t i = i0 + r;
        if (i >= M) break;
        const int h0 = (t - r * cpr) * 8;
        const uint8_t* row = smem + hot_bytes + r * row_bytes;
        const uint16_t* xr = (const uint16_t*)row;
        // the chunk's 8 slot columns as two 16-byte reads
        const int4 c0 = *(const int4*)(hs + h0), c1 = *(const int4*)(hs + h0 + 4);
        const int cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        uint32_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int h = h0 + q;
            const int c = cs[q];
            uint32_t bits = 0;
            if (c >= 0) {
                if (h < n_hot)
                    bits = xr[c];
                else
                    bits = f32_to_bf16_bits(deq_nibble(row + K * 2, row + K * 2 + K / 2, c));
            }
            v[q] = bits;
        }
        uint4 o;
        o.x = v[0] | (v[1] << 16);
        o.y = v[2] | (v[3] << 16);
        o.z = v[4] | (v[5] << 16);
        o.w = v[6] | (v[7] << 16);
        *(uint4*)(a + i * kp + h0) = o;
    }
}

__global__ __launch_bounds__(kThreads) void hcp_gather_w(const uint16_t* __restrict__ w,
                                                         const uint8_t* __restrict__ wqc,
                                                         const uint8_t* __restrict__ wqs,
                                                         const int32_t* __restrict__ hot,
                                                         int n_hot, int64_t N, int64_t K,
                                                         int64_t kp, uint16_t* __restrict__ b,
                                                         int with_q) {
    const int64_t j = (int64_t)blockIdx.x * 64 + (threadIdx.x & 63);
    const int64_t hc = (int64_t)blockIdx.y * (kThreads / 64) + (threadIdx.x >> 6);
    if (j >= N || hc >= kp / 8) return;
    const int h0 = (int)hc * 8;
    uint32_t v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int h = h0 + q;
        uint32_t bits = 0;
        if (h < n_hot) {
            bits = w[(int64_t)hot[h] * N + j];
        } else if (with_q && h < 2 * n_hot) {
            const int c = hot[h - n_hot];
            bits = f32_to_bf16_bits(-deq_nibble(wqc + j * (K / 2), wqs + j * (K / 32), c));
        }
        v[q] = bits;
    }
    uint4 o;
    o.x = v[0] | (v[1] << 16);
    o.y = v[2] | (v[3] << 16);
    o.z = v[4] | (v[5] << 16);
    o.w = v[6] | (v[7] << 16);
    *(uint4*)(b + j * kp + h0) = o;
}

// Row-staged gather of B' = [W_H ; -Wq_H]^T (with_q): a workgroup forms
// JB = 4 consecutive rows j of B'.  Dynamic LDS holds the slot -> column
// table (kp int32), the hot rows' values W[hot[h], j0 .. j0+3] transposed to
// [4][n_hot rounded up to 8] (read 8 bytes per hot row when the rows allow)
// and the 4 K-major code rows (K/2 bytes each) and scale rows (K/32 bytes
// each) of Wq; the output rows then leave as consecutive 16-byte chunks.
// K % 32 == 0.  A hot index outside [0, K) reads as zero.
__global__ __launch_bounds__(kThreads) void hcp_gather_w_rows(
    const uint16_t* __restrict__ w, const uint8_t* __restrict__ wqc,
    const uint8_t* __restrict__ wqs, const int32_t* __restrict__ hot, int n_hot, int64_t N,
    int64_t K, int64_t kp, uint16_t* __restrict__ b, int with_q, int hot_bytes, int wh_bytes) {
    constexpr int JB = kGatherWRows;
    static_assert(JB == 4, "8-byte loads of the hot rows' values");
    extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
    int32_t* hs = (int32_t*)smem;                  // slot -> column (kp entries)
    uint16_t* wh = (uint16_t*)(smem + hot_bytes);  // [JB][hp]: W[hot[h], j0 + jj]
    const int hp = wh_bytes / (2 * JB);            // n_hot rounded up to 8
    uint8_t* cr = smem + hot_bytes + wh_bytes;      // [JB][K/2] codes, then [JB][K/32] scales
    uint8_t* sr = cr + JB * (K / 2);
    const int tid = threadIdx.x;
    const int64_t j0 = (int64_t)blockIdx.x * JB;
    const int nj = (int)std::min<int64_t>(JB, N - j0);
    fill_slot_columns(hs, hot, n_hot, kp, 1, K);
    __syncthreads();
    const bool vec = (N % JB) == 0 && nj == JB;  // 8-byte aligned, whole
    for (int h = tid; h < hp; h += kThreads) {
        const int c = h < n_hot ? hs[h] : -1;
        uint32_t e[JB / 2];
#pragma unroll
        for (int q = 0; q < JB / 2; ++q) e[q] = 0u;
        if (c >= 0) {
            const uint16_t* src = w + (int64_t)c * N + j0;
            if (vec) {
                const uint2 v = *(const uint2*)src;
                e[0] = v.x;
                e[1] = v.y;
            } else {
#pragma unroll
                for (int q = 0; q < JB; ++q)
                    e[q >> 1] |= (q < nj ? (uint32_t)src[q] : 0u) << (16 * (q & 1));
            }
        }
#pragma unroll
        for (int q = 0; q < JB; ++q) wh[q * hp + h] = (uint16_t)(e[q >> 1] >> (16 * (q & 1)));
    }
    if (with_q) {
        const int cw = (int)(K / 2 / 16);
        for (int t = tid; t < nj * cw; t += kThreads) {
            const int jj = t / cw, c = t - jj * cw;
            ((uint4*)(cr + jj * (K / 2)))[c] = ((const uint4*)(wqc + (j0 + jj) * (K / 2)))[c];
        }
        const int sw = (int)(K / 32);
        for (int t = tid; t < nj * sw; t += kThreads) {
            const int jj = t / sw, c = t - jj * sw;
            sr[jj * sw + c] = wqs[(j0 + jj) * sw + c];
        }
    }
    __syncthreads();
    const int cpr = (int)(kp / 8);
    for (int t = tid; t < nj * cpr; t += kThreads) {
        const int jj = t / cpr;
        const int h0 = (t - jj * cpr) * 8;
        const int4 c0 = *(const int4*)(hs + h0), c1 = *(const int4*)(hs + h0 + 4);
        const int cs[8] = {c0.x, c0.y, c0.z, c0.w, c1.x, c1.y, c1.z, c1.w};
        // this row's W values of slots h0 .. h0+7 (read whole when all of
        // them are hot slots)
        uint4 wv = make_uint4(0u, 0u, 0u, 0u);
        if (h0 + 8 <= hp) wv = *(const uint4*)(wh + jj * hp + h0);
        const uint32_t we[4] = {wv.x, wv.y, wv.z, wv.w};
        uint32_t v[8];
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int h = h0 + q;
            const int c = cs[q];
            uint32_t bits = 0;
            if (c >= 0) {
                if (h < n_hot)
                    bits = (we[q >> 1] >> (16 * (q & 1))) & 0xFFFFu;
                else
                    bits = f32_to_bf16_bits(-deq_nibble(cr + jj * (K / 2), sr + jj * (K / 32), c));
            }
            v[q] = bits;
        }
        uint4 o;
        o.x = v[0] | (v[1] << 16);
        o.y = v[2] | (v[3] << 16);
        o.z = v[4] | (v[5] << 16);
        o.w = v[6] | (v[7] << 16);
        *(uint4*)(b + (j0 + jj) * kp + h0) = o;
    }
}

// Gathers the hot operands into the workspace: A' [M, kp] then B' [N, kp]
// (with_q: [X_H | Xq_H], [W_H ; -Wq_H]; else X_H, W_H alone).
static hipError_t gather_hot(int64_t M, int64_t N, int64_t K, const void* x, const uint8_t* xqc,
                             const uint8_t* xqs, const void* w, const uint8_t* wqc,
                             const uint8_t* wqs, const int32_t* hot, int32_t n_hot, void* ws,
                             hipStream_t s, uint16_t** ap_out, uint16_t** bp_out,
                             int with_q = 1) {
    const int64_t kp = with_q ? padded_k(n_hot) : padded_k_split(n_hot);
    uint16_t* ap = (uint16_t*)ws;
    uint16_t* bp = (uint16_t*)((uint8_t*)ws + round_up((size_t)(M * kp * 2), 256));
    {
        // rows staged whole in LDS when a row and the hot list fit in 40 KB;
        // about 8 KB of rows per workgroup (1 to 4): the workgroups resident
        // on a compute unit, not the rows each stages, keep its loads in
        // flight (13B-shaped X, 13 KB rows: 83 -> 70 us with one row per
        // workgroup instead of two; 140 us with four)
        const int64_t hot_bytes = kp * 4;  // the slot -> column table
        const int64_t row_bytes = (int64_t)round_up((size_t)(K * 2 + (with_q ? K / 2 + K / 32 : 0)), 16);
        constexpr int64_t kLdsBudget = 40 * 1024;
        if (hot_bytes + row_bytes <= kLdsBudget) {
            const int rpw = (int)std::max<int64_t>(
                1, std::min<int64_t>({4, 8192 / row_bytes, (kLdsBudget - hot_bytes) / row_bytes}));
            const size_t lds = (size_t)(hot_bytes + rpw * row_bytes);
            dim3 grid((unsigned)((M + rpw - 1) / rpw));
            FP4Q_LAUNCH((hcp_gather_x_rows), grid, kThreads, lds, s, (const uint16_t*)x, xqc, xqs, hot, n_hot,
                                                          M, K, kp, ap, with_q, rpw, (int)hot_bytes,
                                                          (int)row_bytes);
        } else {
            const int64_t total = M * (kp / 8);
            dim3 grid((unsigned)((total + kThreads - 1) / kThreads));
            FP4Q_LAUNCH((hcp_gather_x), grid, kThreads, 0, s, (const uint16_t*)x, xqc, xqs, hot, n_hot, M, K,
                                                   kp, ap, with_q);
        }
    }
    {
        // four rows of B' per workgroup, staged in LDS, when they fit in 40 KB
        // (with_q only: W's hot rows alone are read coalesced by the kernel below)
        constexpr int JB = kGatherWRows;
        const int64_t hot_bytes = kp * 4;
        const int64_t wh_bytes = (int64_t)round_up((size_t)n_hot, 8) * 2 * JB;
        const int64_t q_bytes = JB * (K / 2 + K / 32);
        if (with_q && hot_bytes + wh_bytes + q_bytes <= 40 * 1024) {
            dim3 grid((unsigned)((N + JB - 1) / JB));
            FP4Q_LAUNCH((hcp_gather_w_rows), grid, kThreads, (size_t)(hot_bytes + wh_bytes + q_bytes), s,
                (const uint16_t*)w, wqc, wqs, hot, n_hot, N, K, kp, bp, with_q, (int)hot_bytes,
                (int)wh_bytes);
        } else {
            dim3 grid((unsigned)((N + 63) / 64), (unsigned)((kp / 8 + 3) / 4));
            FP4Q_LAUNCH((hcp_gather_w), grid, kThreads, 0, s, (const uint16_t*)w, wqc, wqs, hot, n_hot, N, K,
                                                   kp, bp, with_q);
        }
    }
    *ap_out = ap;
    *bp_out = bp;
    return hipGetLastError();
}

// ---------------------------------------------------------------------------
// Library-owned scratch for fp4q_hcp_residual_add_noalloc (callers that
// cannot allocate): the gathered hot operands A' [M, kp] and B' [N, kp] live
// in this file-scope device array instead of a caller workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  In host
// code `scratch` is only a stand-in for the symbol: its device address is
// taken once per device with hipGetSymbolAddress and only that address is
// ever passed to kernels.  The gathers write every element of A' and B'
// (padding included), so nothing has to be cleared between calls; calls
// that overlap on one GPU share the array and race.
static __device__ __align__(256) uint8_t scratch[kHcpStaticScratchBytes];

static std::mutex g_scratch_mu;
static void* g_scratch_dev[kMaxDevices];  // device address of `scratch`, per device

hipError_t hcp_static_scratch(void** out) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    if (dev < 0 || dev >= kMaxDevices) return hipErrorInvalidDevice;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_dev[dev]) {
        void* p = nullptr;
        e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));  // with `dev` current
        if (e != hipSuccess) return e;
        g_scratch_dev[dev] = p;
    }
    *out = g_scratch_dev[dev];
    return hipSuccess;
}

hipError_t launch_hcp(int64_t M, int64_t N, int64_t K, const void* x, const uint8_t* xqc,
                      const uint8_t* xqs, const void* w, const uint8_t* wqc, const uint8_t* wqs,
                      const int32_t* hot, int32_t n_hot, float* y, void* ws, hipStream_t s) {
    if (n_hot <= 0) return hipSuccess;
    uint16_t *ap, *bp;
    hipError_t e = gather_hot(M, N, K, x, xqc, xqs, w, wqc, wqs, hot, n_hot, ws, s, &ap, &bp);
    if (e != hipSuccess) return e;
    return launch_gemm_bf16_accum(M, N, padded_k(n_hot), ap, bp, y, N, s);
}

hipError_t launch_gemm_hcp(int64_t M, int64_t N, int64_t K, const void* x, const uint8_t* xqc,
                           const uint8_t* xqs, const void* w, const uint8_t* wqc,
                           const uint8_t* wqs, const int32_t* hot, int32_t n_hot, float* y,
                           int64_t ldy, void* ws, hipStream_t s) {
    if (n_hot <= 0) return launch_gemm_fp4(M, N, K, xqc, xqs, wqc, wqs, y, F32, ldy, false, s);
    uint16_t *ap, *bp;
    hipError_t e = gather_hot(M, N, K, x, xqc, xqs, w, wqc, wqs, hot, n_hot, ws, s, &ap, &bp);
    if (e != hipSuccess) return e;
    return launch_gemm_fp4_hot(M, N, K, xqc, xqs, wqc, wqs, ap, bp, padded_k(n_hot), y, ldy, s);
}

hipError_t launch_gemm_hcp_split(int64_t M, int64_t N, int64_t K, const void* x,
                                 const uint8_t* xqc, const uint8_t* xqs, const void* w,
                                 const uint8_t* wqc, const uint8_t* wqs, const int32_t* hot,
                                 int32_t n_hot, float* y, int64_t ldy, void* ws, hipStream_t s) {
    if (n_hot <= 0) return launch_gemm_fp4(M, N, K, xqc, xqs, wqc, wqs, y, F32, ldy, false, s);
    uint16_t *ap, *bp;
    hipError_t e =
        gather_hot(M, N, K, x, xqc, xqs, w, wqc, wqs, hot, n_hot, ws, s, &ap, &bp, /*with_q=*/0);
    if (e != hipSuccess) return e;
    return launch_gemm_fp4_hot(M, N, K, xqc, xqs, wqc, wqs, ap, bp, padded_k_split(n_hot), y, ldy,
                               s);
}

}  // namespace fp4q
