// MXFP4 dequantizer (the DQ half of the QDQ node pair of the MXFP4 tutorial
// page, sec. 6.1): value(code) * 2^(byte - 127), written as bf16 or fp32.
//
// HBM-streaming and fully flat: the codes, scales and output are dense, so
// chunk g of 8 elements reads code word g, scale byte 8g/block, and writes
// output elements [8g, 8g+8) -- no index arithmetic beyond a shift.  The
// gfx950 scaled conversion from FP4 produces each pair exactly (the product
// of an E2M1 value and a power of two); byte 0xFF (NaN scale) forces NaN.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

static constexpr int kThreads = 256;
static constexpr int kUnroll = 4;

template <int OUT_BF16, int LOG2_G>
__global__ __launch_bounds__(kThreads) void dequantize_kernel(const uint32_t* __restrict__ codes,
                                                              const uint8_t* __restrict__ scales,
                                                              uint32_t total_chunks,
                                                              void* __restrict__ y) {
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = blockIdx.x * (kThreads / 64) + (threadIdx.x >> 6);
    const uint32_t base = wave * 64u * kUnroll;
    uint32_t cw[kUnroll], sb[kUnroll];
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t g = base + u * 64u + lane;
        const uint32_t gg = g < total_chunks ? g : 0u;
        cw[u] = codes[gg];
        sb[u] = scales[gg >> LOG2_G];
    }
#pragma unroll
    for (int u = 0; u < kUnroll; ++u) {
        const uint32_t g = base + u * 64u + lane;
        if (g >= total_chunks) continue;
        const float sc = e8m0_scale_f32(sb[u]);
        const bool nan_blk = sb[u] == 0xFFu;
        if (OUT_BF16) {
            uint4 o;
            o.x = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[u], sc, 0));
            o.y = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[u], sc, 1));
            o.z = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[u], sc, 2));
            o.w = __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp4(cw[u], sc, 3));
            if (nan_blk) o.x = o.y = o.z = o.w = 0x7FC07FC0u;
            store_nt((uint4*)y + g, o);
        } else {
            f32x2_t a = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], sc, 0);
            f32x2_t b = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], sc, 1);
            f32x2_t c = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], sc, 2);
            f32x2_t d = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(cw[u], sc, 3);
            uint4 o0, o1;
            o0.x = as_u32(a.x);
            o0.y = as_u32(a.y);
            o0.z = as_u32(b.x);
            o0.w = as_u32(b.y);
            o1.x = as_u32(c.x);
            o1.y = as_u32(c.y);
            o1.z = as_u32(d.x);
            o1.w = as_u32(d.y);
            if (nan_blk) {
                o0.x = o0.y = o0.z = o0.w = 0x7FC00000u;
                o1 = o0;
            }
            store_nt((uint4*)y + 2 * g, o0);
            store_nt((uint4*)y + 2 * g + 1, o1);
        }
    }
}

template <int OUT_BF16>
static void dq_dispatch(int block, dim3 grid, hipStream_t s, const uint32_t* c, const uint8_t* sc,
                        uint32_t tc, void* y) {
    switch (block) {
        case 16: FP4Q_LAUNCH((dequantize_kernel<OUT_BF16, 1>), grid, kThreads, 0, s, c, sc, tc, y); break;
        case 32: FP4Q_LAUNCH((dequantize_kernel<OUT_BF16, 2>), grid, kThreads, 0, s, c, sc, tc, y); break;
        case 64: FP4Q_LAUNCH((dequantize_kernel<OUT_BF16, 3>), grid, kThreads, 0, s, c, sc, tc, y); break;
        default: FP4Q_LAUNCH((dequantize_kernel<OUT_BF16, 4>), grid, kThreads, 0, s, c, sc, tc, y); break;
    }
}

hipError_t launch_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                             int block, void* y, int ydtype, hipStream_t s) {
    const uint32_t tc = (uint32_t)(rows * k / 8);
    const uint32_t per_wg = 64u * kUnroll * (kThreads / 64);
    dim3 grid((tc + per_wg - 1) / per_wg);
    if (ydtype == BF16)
        dq_dispatch<1>(block, grid, s, (const uint32_t*)codes, scales, tc, y);
    else
        dq_dispatch<0>(block, grid, s, (const uint32_t*)codes, scales, tc, y);
    return hipGetLastError();
}

}  // namespace fp4q
