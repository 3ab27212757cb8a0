// Random Hadamard transform fused into block-32 quantisation (the recipe of
// the outlier-dynamics page, sec. 4.1, transforms backward operands before
// quantising them).  Along the block axis, each group of 32 values becomes
//
//   y = 2^-2.5 * H32 * D * x,
//
// D = diag(+-1) from a caller-given sign mask over the axis, H32 the natural
// (Sylvester) order Hadamard matrix.  2^-2.5 * H32 is orthogonal, so a GEMM
// whose two operands are transformed along their shared contraction axis
// with the same signs keeps its product.  The transform is evaluated in fp32
// as butterflies (a, b) -> (a + b, a - b) on pairs (i, i + s) with bit s of i
// clear, s = 1, 2, 4, 8, 16, then the product by fl32(2^-2.5): five rounded
// levels of additions and two roundings for the constant, so every value is
// within 8 * 2^-24 * 2^-2.5 * sum|x| of the exact y, and the fixed order makes
// the values the codes are decided on deterministic run to run.  The block's
// scale and codes then follow the ordinary quantiser (nearest-even or
// stochastic with counter r*cols + c + offset).
//
//  * rht_row_kernel: a thread holds 8 consecutive values of a row, four
//    lanes one group: strides 1..4 in registers, 8 and 16 across the quad by
//    DPP; codes as the ROW quantiser lays them out.
//  * rht_col_kernel: a thread holds two adjacent columns x 32 rows (one group
//    per column) in registers, all five strides in registers, one group down
//    the rows per workgroup unless the grid's y extent needs more;
//    stochastic bits come from a shared LDS fill.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

static constexpr int kRhtThreads = 256;
static constexpr uint32_t kRhtC = 0x3E3504F3u;  // 2^-2.5 rounded to fp32

__device__ __forceinline__ float dpp_quad(float v, int ctrl_is_xor2) {
    const int iv = __builtin_bit_cast(int, v);
    const int r = ctrl_is_xor2 ? __builtin_amdgcn_update_dpp(0, iv, 0x4E, 0xF, 0xF, false)
                               : __builtin_amdgcn_update_dpp(0, iv, 0xB1, 0xF, 0xF, false);
    return __builtin_bit_cast(float, r);
}

// In-register butterflies over strides 1, 2, 4 of 8 consecutive values.
__device__ __forceinline__ void fwht8(float v[8]) {
#pragma unroll
    for (int s = 1; s < 8; s <<= 1)
#pragma unroll
        for (int i = 0; i < 8; ++i)
            if (!(i & s)) {
                const float a = v[i], b = v[i + s];
                v[i] = a + b;
                v[i + s] = a - b;
            }
}

template <int SR>
__global__ __launch_bounds__(kRhtThreads) void rht_row_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const uint32_t* __restrict__ signs, uint32_t k0, uint32_t k1, uint64_t off,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    const int64_t cpr = cols / 8;  // chunks per row (a multiple of 4)
    const int64_t g = (int64_t)blockIdx.x * kRhtThreads + threadIdx.x;
    if (g >= rows * cpr) return;  // whole quads leave together
    const int64_t r = g / cpr;
    const int64_t c0 = (g - r * cpr) * 8;
    const int L = threadIdx.x & 3;
    const uint4 w = *(const uint4*)(x + r * ld + c0);
    const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
    float v[8] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1),
                  bf16_lo(w2), bf16_hi(w2), bf16_lo(w3), bf16_hi(w3)};
    const uint32_t sb = (signs[c0 >> 5] >> (c0 & 31)) & 0xFFu;
#pragma unroll
    for (int e = 0; e < 8; ++e)
        if ((sb >> e) & 1u) v[e] = -v[e];
    fwht8(v);
    // stride 8: lanes L, L^1; stride 16: lanes L, L^2 (lower lane a + b,
    // upper lane a - b with a the lower lane's value)
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float p = dpp_quad(v[e], 0);
        v[e] = (L & 1) ? p - v[e] : v[e] + p;
    }
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const float p = dpp_quad(v[e], 1);
        v[e] = (L & 2) ? p - v[e] : v[e] + p;
    }
    const float cc = as_f32(kRhtC);
    uint32_t amax = 0;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        v[e] = v[e] * cc;
        amax = max(amax, as_u32(v[e]) & 0x7FFFFFFFu);
    }
    amax = group_max_u32<4>(amax);
    const bool nf = amax >= 0x7F800000u;
    const uint32_t byte = nf ? 0xFFu : e8m0_from_amax(amax);
    const float sc = e8m0_scale_f32(nf ? 0u : byte);
    uint32_t packed = 0;
    if (!SR) {
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[0], v[1], sc, 0);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[2], v[3], sc, 1);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[4], v[5], sc, 2);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[6], v[7], sc, 3);
    } else {
        uint32_t wr[4];
        sr_words8((uint64_t)r * (uint64_t)cols + (uint64_t)c0 + off, k0, k1, wr);
        packed = sr_pack8(v, sc, wr);
    }
    ((uint32_t*)codes)[g] = nf ? 0u : packed;
    if (L == 0) scales[g >> 2] = (uint8_t)byte;
}

__device__ __forceinline__ void fwht32(float v[32]) {
#pragma unroll
    for (int s = 1; s < 32; s <<= 1)
#pragma unroll
        for (int i = 0; i < 32; ++i)
            if (!(i & s)) {
                const float a = v[i], b = v[i + s];
                v[i] = a + b;
                v[i + s] = a - b;
            }
}

// Codes (16 bytes, rows 2k low / 2k + 1 high nibble) and scale of one column
// group already transformed and scaled by c; u[i] are the SR bits of row i.
template <int SR>
__device__ __forceinline__ uint4 col_group_codes(const float v[32], const uint32_t* u,
                                                 uint32_t& byte) {
    uint32_t amax = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) amax = max(amax, as_u32(v[i]) & 0x7FFFFFFFu);
    const bool nf = amax >= 0x7F800000u;
    byte = nf ? 0xFFu : e8m0_from_amax(amax);
    const float sc = e8m0_scale_f32(nf ? 0u : byte);
    uint32_t wv[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        uint32_t packed = 0;
        if (!SR) {
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[8 * q + 0], v[8 * q + 1], sc, 0);
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[8 * q + 2], v[8 * q + 3], sc, 1);
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[8 * q + 4], v[8 * q + 5], sc, 2);
            packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, v[8 * q + 6], v[8 * q + 7], sc, 3);
        } else {
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const int i = 8 * q + 2 * k;
                packed |= sr_pair(v[i], v[i + 1], sc, u[i] << 16, u[i + 1] << 15) << (8 * k);
            }
        }
        wv[q] = nf ? 0u : packed;
    }
    return make_uint4(wv[0], wv[1], wv[2], wv[3]);
}

// Stochastic rounding takes its bits from LDS: per group row the workgroup
// fills 32 rows x 512 columns of 16-bit lanes with one Philox call per 8
// consecutive positions (the ROW quantiser's lanes), stored as [row][column
// pair] words, low half the even column, so each thread reads its pair's bits
// with one 32-bit access per row.
template <int SR>
__global__ __launch_bounds__(kRhtThreads) void rht_col_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld,
    const uint32_t* __restrict__ signs, uint32_t k0, uint32_t k1, uint64_t off, int rb_per,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales) {
    __shared__ __align__(16) uint32_t rnd[SR ? 32 * kRhtThreads : 1];
    const int tid = threadIdx.x;
    const int64_t nb = rows / 32;
    const uint32_t ny = (uint32_t)((nb + rb_per - 1) / rb_per);
    // Workgroups are dealt to the eight XCDs in turn; remap so that each XCD
    // takes a contiguous run of tiles ordered by column block, row groups
    // fastest: the 16-byte code pieces and scale bytes that consecutive row
    // groups write into one line of a column's output then meet in that
    // XCD's L2 and leave it as whole lines (dY's codes: 3.2x the algorithmic
    // bytes written before).
    uint32_t tile = blockIdx.x;
    {
        const uint32_t full = (gridDim.x / 8) * 8;
        if (tile < full) tile = (tile % 8) * (full / 8) + tile / 8;
    }
    const uint32_t xblk = tile / ny, yblk = tile - xblk * ny;
    const int64_t cbase = (int64_t)xblk * kRhtThreads * 2;
    const int64_t c = cbase + 2 * tid;
    const bool cok = c < cols;  // no early exit: the workgroup meets at barriers
    const float cc = as_f32(kRhtC);
    for (int t = 0; t < rb_per; ++t) {
        const int64_t b = (int64_t)yblk * rb_per + t;
        if (b >= nb) break;  // uniform over the workgroup
        const int64_t r0 = b * 32;
        // this group's 32 rows are loaded first, so their latency passes
        // while the stochastic bits are filled
        uint32_t xw[32];
#pragma unroll
        for (int i = 0; i < 32; ++i)
            xw[i] = cok ? *(const uint32_t*)(x + (r0 + i) * ld + c) : 0u;
        if (SR) {
            __syncthreads();  // the previous group row's bits are consumed
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int chunk = tid + kRhtThreads * j;  // 32 rows x 64 chunks of 8
                const int i = chunk >> 6, q = chunk & 63;
                uint32_t wr[4];
                sr_words8((uint64_t)(r0 + i) * (uint64_t)cols + (uint64_t)(cbase + 8 * q) + off, k0,
                          k1, wr);
                *(uint4*)&rnd[i * kRhtThreads + 4 * q] = make_uint4(wr[0], wr[1], wr[2], wr[3]);
            }
            __syncthreads();
        }
        if (!cok) continue;
        float v0[32], v1[32];
        const uint32_t sg = signs[b];
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            const uint32_t w = xw[i];
            const float lo = bf16_lo(w), hi = bf16_hi(w);
            const bool neg = (sg >> i) & 1u;
            v0[i] = neg ? -lo : lo;
            v1[i] = neg ? -hi : hi;
        }
        fwht32(v0);
        fwht32(v1);
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            v0[i] = v0[i] * cc;
            v1[i] = v1[i] * cc;
        }
        uint32_t u0[SR ? 32 : 1], u1[SR ? 32 : 1];
        if (SR) {
#pragma unroll
            for (int i = 0; i < 32; ++i) {
                const uint32_t w = rnd[i * kRhtThreads + tid];
                u0[i] = w & 0xFFFFu;
                u1[i] = w >> 16;
            }
        }
        uint32_t byte0, byte1;
        const uint4 q0 = col_group_codes<SR>(v0, u0, byte0);
        const uint4 q1 = col_group_codes<SR>(v1, u1, byte1);
        *(uint4*)(codes + c * (rows / 2) + r0 / 2) = q0;
        *(uint4*)(codes + (c + 1) * (rows / 2) + r0 / 2) = q1;
        scales[c * nb + b] = (uint8_t)byte0;
        scales[(c + 1) * nb + b] = (uint8_t)byte1;
    }
}

hipError_t launch_quantize_rht(const void* x, int64_t rows, int64_t cols, int64_t ld, bool col,
                               const uint32_t* signs, bool sr, uint64_t seed, uint64_t off,
                               uint8_t* codes, uint8_t* scales, hipStream_t s) {
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const uint16_t* xb = (const uint16_t*)x;
    if (!col) {
        const int64_t chunks = rows * (cols / 8);
        const dim3 grid((unsigned)((chunks + kRhtThreads - 1) / kRhtThreads));
        if (sr)
            FP4Q_LAUNCH((rht_row_kernel<1>), grid, kRhtThreads, 0, s, xb, rows, cols, ld, signs, k0, k1, off,
                                                          codes, scales);
        else
            FP4Q_LAUNCH((rht_row_kernel<0>), grid, kRhtThreads, 0, s, xb, rows, cols, ld, signs, k0, k1, off,
                                                          codes, scales);
    } else {
        // one group per thread down the rows (the grid's size allowing):
        // measured on MI355X, dY 8192 x 5632 SR 50.1 / 51.0 / 56.4 us with
        // 1 / 2 / 4 groups per thread, X 8192 x 2048 14.8 / 17.4 / 17.0 us
        // (the longer code runs per column of more groups do not pay for the
        // lost parallelism)
        const int64_t gx = (cols / 2 + kRhtThreads - 1) / kRhtThreads, nb = rows / 32;
        int rb = 1;
        while (gx * ((nb + rb - 1) / rb) > 0x7FFFFFFF) rb <<= 1;
        const dim3 grid((unsigned)(gx * ((nb + rb - 1) / rb)));
        if (sr)
            FP4Q_LAUNCH((rht_col_kernel<1>), grid, kRhtThreads, 0, s, xb, rows, cols, ld, signs, k0, k1, off,
                                                          rb, codes, scales);
        else
            FP4Q_LAUNCH((rht_col_kernel<0>), grid, kRhtThreads, 0, s, xb, rows, cols, ld, signs, k0, k1, off,
                                                          rb, codes, scales);
    }
    return hipGetLastError();
}

}  // namespace fp4q
