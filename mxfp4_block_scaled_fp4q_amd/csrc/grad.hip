// Backward gradient estimators of the quantizer Q.
//
//  * STE: dQ/dx is taken as 1 (MXFP4 tutorial page, sec. 3.1): out = grad,
//    converted to the output dtype.
//  * DGE: the differentiable estimator of the MSRA FP4-training summary page,
//    sec. 二 -- Q is replaced on each quantisation interval of width delta by
//    f = delta/2 (1 + sign(u) |u|^(1/k)), u = 2 t / delta - 1 (t = offset from
//    the interval's lower end), whose derivative (1/k)|u|^(1/k - 1) is clamped
//    at clamp_max (3.0 on that page).  out = grad * d.  The interval is found
//    on x's own E2M1 grid: the block scale is recomputed here from x with the
//    same block and axis as its quantisation.  Beyond the grid (|x|/s > 6,
//    saturated) the estimator falls back to STE (d = 1).
//
// Interval arithmetic: with m = |x|/s and E = max(biased exponent(m), 127),
// q = m * 2^(128 - E) maps every E2M1 interval onto a unit interval
// [floor(q), floor(q) + 1), so u = 2 (q - floor(q)) - 1 exactly; |u|^(p) is
// computed as exp2(p * log2|u|) on the hardware transcendental units (|u| = 0
// gives +inf, i.e. the clamp).
//
// HBM-streaming: ROW mirrors the ROW quantizer (lanes own 8 elements, DPP
// amax across the block's lanes); COL mirrors the COL quantizer (lanes own 8
// adjacent columns x 8 rows, DPP amax across the block's lanes).
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

static constexpr int kThreads = 256;

template <int BF16>
__device__ __forceinline__ void load8(const void* p, int64_t e0, float (&f)[8]) {
    if (BF16) {
        const uint4 v = *(const uint4*)((const uint16_t*)p + e0);
        f[0] = bf16_lo(v.x);
        f[1] = bf16_hi(v.x);
        f[2] = bf16_lo(v.y);
        f[3] = bf16_hi(v.y);
        f[4] = bf16_lo(v.z);
        f[5] = bf16_hi(v.z);
        f[6] = bf16_lo(v.w);
        f[7] = bf16_hi(v.w);
    } else {
        const uint4* q = (const uint4*)((const float*)p + e0);
        const uint4 a = q[0], b = q[1];
        f[0] = as_f32(a.x);
        f[1] = as_f32(a.y);
        f[2] = as_f32(a.z);
        f[3] = as_f32(a.w);
        f[4] = as_f32(b.x);
        f[5] = as_f32(b.y);
        f[6] = as_f32(b.z);
        f[7] = as_f32(b.w);
    }
}

template <int BF16>
__device__ __forceinline__ void store8(void* p, int64_t e0, const float (&f)[8]) {
    if (BF16) {
        uint4 v;
        v.x = pack_bf16x2(f[0], f[1]);
        v.y = pack_bf16x2(f[2], f[3]);
        v.z = pack_bf16x2(f[4], f[5]);
        v.w = pack_bf16x2(f[6], f[7]);
        store_nt((uint4*)((uint16_t*)p + e0), v);
    } else {
        uint4* q = (uint4*)((float*)p + e0);
        store_nt(q, make_uint4(as_u32(f[0]), as_u32(f[1]), as_u32(f[2]), as_u32(f[3])));
        store_nt(q + 1, make_uint4(as_u32(f[4]), as_u32(f[5]), as_u32(f[6]), as_u32(f[7])));
    }
}

// ---------------------------------------------------------------------------
// STE: a converting copy.  8 elements per lane per step; a scalar tail.
// ---------------------------------------------------------------------------
template <int GB, int OB>
__global__ __launch_bounds__(kThreads) void ste_kernel(const void* __restrict__ g, int64_t n,
                                                       void* __restrict__ out) {
    const int64_t nchunks = n / 8;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    for (int64_t c = (int64_t)blockIdx.x * kThreads + threadIdx.x; c < nchunks; c += stride) {
        float f[8];
        load8<GB>(g, c * 8, f);
        store8<OB>(out, c * 8, f);
    }
    if (blockIdx.x == 0 && threadIdx.x < (n & 7)) {
        const int64_t i = nchunks * 8 + threadIdx.x;
        const float v = GB ? bf16_lo(((const uint16_t*)g)[i]) : ((const float*)g)[i];
        if (OB)
            ((uint16_t*)out)[i] = (uint16_t)f32_to_bf16_bits(v);
        else
            ((float*)out)[i] = v;
    }
}

// ---------------------------------------------------------------------------
// DGE, ROW blocks
// ---------------------------------------------------------------------------
template <int XB, int GB, int OB, int BLOCK>
__global__ __launch_bounds__(kThreads) void dge_row_kernel(const void* __restrict__ x,
                                                           const void* __restrict__ g,
                                                           uint32_t total_chunks,
                                                           void* __restrict__ out, DgeParams P) {
    constexpr int G = BLOCK / 8;
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const uint32_t gi = wave * 64u + lane;
    const bool valid = gi < total_chunks;
    const int64_t e0 = (int64_t)(valid ? gi : 0u) * 8;
    float xf[8], gf[8];
    load8<XB>(x, e0, xf);
    load8<GB>(g, e0, gf);
    uint32_t amax = 0;
#pragma unroll
    for (int j = 0; j < 8; ++j) amax = max(amax, as_u32(xf[j]) & 0x7FFFFFFFu);
    amax = valid ? amax : 0u;
    amax = group_max_u32<G>(amax);
    const bool nf = amax >= 0x7F800000u;
    const float inv = e8m0_inv_scale_f32(nf ? 0u : e8m0_from_amax(amax));
    float o[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float d = nf ? __builtin_nanf("") : dge_factor(xf[j], inv, P);
        o[j] = gf[j] * d;
    }
    if (valid) store8<OB>(out, e0, o);
}

// ---------------------------------------------------------------------------
// DGE, COL blocks: a lane owns 8 adjacent columns x 8 consecutive rows; the
// block/8 lanes of one column block are adjacent and reduce the column amax
// with DPP, as in the COL quantizer.  x stays in registers as raw bits
// between the amax and the gradient pass.
// ---------------------------------------------------------------------------
template <int XB, int GB, int OB, int BLOCK>
__global__ __launch_bounds__(kThreads) void dge_col_kernel(const void* __restrict__ x,
                                                           const void* __restrict__ g,
                                                           int64_t rows, int64_t cols,
                                                           void* __restrict__ out, DgeParams P,
                                                           int64_t ncg, int64_t nrb,
                                                           int64_t n_cchunks) {
    constexpr int XW = XB ? 4 : 8;  // 32-bit words per 8 x values
    constexpr int G = BLOCK / 8;
    constexpr int CG_PER_WAVE = 64 / G;
    const int lane = threadIdx.x & 63;
    const int64_t wave = (int64_t)blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    if (wave >= nrb * n_cchunks) return;  // whole wave
    const int64_t rb = wave / n_cchunks;
    const int64_t cg = (wave - rb * n_cchunks) * CG_PER_WAVE + lane / G;
    const int rq = lane % G;
    const bool cg_ok = cg < ncg;
    const int64_t c0 = (cg_ok ? cg : 0) * 8;
    const bool full = cg_ok && ((cols & 7) == 0) && (c0 + 8 <= cols);
    const int64_t r0 = rb * BLOCK + rq * 8;

    uint32_t xs[8][XW];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = r0 + i;
        if (full) {
            const uint4* q = XB ? (const uint4*)((const uint16_t*)x + r * cols + c0)
                                : (const uint4*)((const float*)x + r * cols + c0);
            const uint4 a = q[0];
            xs[i][0] = a.x;
            xs[i][1] = a.y;
            xs[i][2] = a.z;
            xs[i][3] = a.w;
            if (!XB) {
                const uint4 b = q[1];
                xs[i][4 % XW] = b.x;
                xs[i][5 % XW] = b.y;
                xs[i][6 % XW] = b.z;
                xs[i][7 % XW] = b.w;
            }
        } else {
            uint32_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t c = c0 + j;
                e[j] = (cg_ok && c < cols) ? (XB ? (uint32_t)((const uint16_t*)x)[r * cols + c]
                                                 : ((const uint32_t*)x)[r * cols + c])
                                           : 0u;
            }
#pragma unroll
            for (int j = 0; j < XW; ++j) xs[i][j] = XB ? (e[2 * j] | (e[2 * j + 1] << 16)) : e[j];
        }
    }
    auto xbits = [&](int i, int j) -> uint32_t {
        if (XB) return (j & 1) ? (xs[i][j >> 1] & 0xFFFF0000u) : (xs[i][j >> 1] << 16);
        return xs[i][j];
    };
    float inv[8];
    bool nf[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) m = max(m, xbits(i, j) & 0x7FFFFFFFu);
        m = group_max_u32<G>(m);
        nf[j] = m >= 0x7F800000u;
        inv[j] = e8m0_inv_scale_f32(nf[j] ? 0u : e8m0_from_amax(m));
    }
    if (!cg_ok) return;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int64_t r = r0 + i;
        float gf[8], o[8];
        if (full) {
            load8<GB>(g, r * cols + c0, gf);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t c = c0 + j;
                gf[j] = c < cols ? (GB ? bf16_lo(((const uint16_t*)g)[r * cols + c])
                                       : ((const float*)g)[r * cols + c])
                                 : 0.0f;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            const float d = nf[j] ? __builtin_nanf("") : dge_factor(as_f32(xbits(i, j)), inv[j], P);
            o[j] = gf[j] * d;
        }
        if (full) {
            store8<OB>(out, r * cols + c0, o);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int64_t c = c0 + j;
                if (c < cols) {
                    if (OB)
                        ((uint16_t*)out)[r * cols + c] = (uint16_t)f32_to_bf16_bits(o[j]);
                    else
                        ((float*)out)[r * cols + c] = o[j];
                }
            }
        }
    }
}

hipError_t launch_ste(const void* g, int gdtype, int64_t n, void* out, int odtype, hipStream_t s) {
    const int64_t nchunks = n / 8;
    int64_t wgs = (nchunks + kThreads - 1) / kThreads;
    if (wgs > 65536) wgs = 65536;
    if (wgs < 1) wgs = 1;
    dim3 grid((unsigned)wgs);
    if (gdtype == BF16 && odtype == BF16) FP4Q_LAUNCH((ste_kernel<1, 1>), grid, kThreads, 0, s, g, n, out);
    else if (gdtype == BF16) FP4Q_LAUNCH((ste_kernel<1, 0>), grid, kThreads, 0, s, g, n, out);
    else if (odtype == BF16) FP4Q_LAUNCH((ste_kernel<0, 1>), grid, kThreads, 0, s, g, n, out);
    else FP4Q_LAUNCH((ste_kernel<0, 0>), grid, kThreads, 0, s, g, n, out);
    return hipGetLastError();
}

template <int XB, int GB, int OB>
static void dge_dispatch(const void* x, const void* g, int64_t rows, int64_t cols, int block,
                         int axis, void* out, DgeParams P, hipStream_t s) {
    if (axis == 0) {
        const uint32_t tc = (uint32_t)(rows * cols / 8);
        dim3 grid((tc + kThreads - 1) / kThreads);
        switch (block) {
            case 16: FP4Q_LAUNCH((dge_row_kernel<XB, GB, OB, 16>), grid, kThreads, 0, s, x, g, tc, out, P); break;
            case 32: FP4Q_LAUNCH((dge_row_kernel<XB, GB, OB, 32>), grid, kThreads, 0, s, x, g, tc, out, P); break;
            case 64: FP4Q_LAUNCH((dge_row_kernel<XB, GB, OB, 64>), grid, kThreads, 0, s, x, g, tc, out, P); break;
            default: FP4Q_LAUNCH((dge_row_kernel<XB, GB, OB, 128>), grid, kThreads, 0, s, x, g, tc, out, P); break;
        }
    } else {
        const int64_t ncg = (cols + 7) / 8;
        const int64_t nrb = rows / block;
        const int64_t cgw = 64 / (block / 8);
        const int64_t ncc = (ncg + cgw - 1) / cgw;
        dim3 grid((unsigned)((nrb * ncc + 3) / 4));
        switch (block) {
            case 16: FP4Q_LAUNCH((dge_col_kernel<XB, GB, OB, 16>), grid, kThreads, 0, s, x, g, rows, cols, out, P, ncg, nrb, ncc); break;
            case 32: FP4Q_LAUNCH((dge_col_kernel<XB, GB, OB, 32>), grid, kThreads, 0, s, x, g, rows, cols, out, P, ncg, nrb, ncc); break;
            case 64: FP4Q_LAUNCH((dge_col_kernel<XB, GB, OB, 64>), grid, kThreads, 0, s, x, g, rows, cols, out, P, ncg, nrb, ncc); break;
            default: FP4Q_LAUNCH((dge_col_kernel<XB, GB, OB, 128>), grid, kThreads, 0, s, x, g, rows, cols, out, P, ncg, nrb, ncc); break;
        }
    }
}

hipError_t launch_dge(const void* x, int xdtype, const void* g, int gdtype, int64_t rows,
                      int64_t cols, int block, int axis, float k, float clamp_max, void* out,
                      int odtype, hipStream_t s) {
    DgeParams P;
    P.invk = 1.0f / k;
    P.p = 1.0f / k - 1.0f;
    P.clamp_max = clamp_max;
    P.k_one = (k == 1.0f);
    const int code = (xdtype == BF16) * 4 + (gdtype == BF16) * 2 + (odtype == BF16);
    switch (code) {
        case 0: dge_dispatch<0, 0, 0>(x, g, rows, cols, block, axis, out, P, s); break;
        case 1: dge_dispatch<0, 0, 1>(x, g, rows, cols, block, axis, out, P, s); break;
        case 2: dge_dispatch<0, 1, 0>(x, g, rows, cols, block, axis, out, P, s); break;
        case 3: dge_dispatch<0, 1, 1>(x, g, rows, cols, block, axis, out, P, s); break;
        case 4: dge_dispatch<1, 0, 0>(x, g, rows, cols, block, axis, out, P, s); break;
        case 5: dge_dispatch<1, 0, 1>(x, g, rows, cols, block, axis, out, P, s); break;
        case 6: dge_dispatch<1, 1, 0>(x, g, rows, cols, block, axis, out, P, s); break;
        default: dge_dispatch<1, 1, 1>(x, g, rows, cols, block, axis, out, P, s); break;
    }
    return hipGetLastError();
}

}  // namespace fp4q
