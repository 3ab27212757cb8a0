// Two-dimensional block scaling: one E8M0 scale per 32 x 32 square of a bf16
// matrix (the recipe of the outlier-dynamics page, sec. 4.1, scales its
// backward operands in 2D blocks).  The square is MXFP4's 32-element block in
// both directions, the granularity at which the gfx950 scaled MFMA takes
// scales along K, so the one set of codes is written twice: in the ROW layout
// (blocks along columns; the operand of a GEMM contracting over columns) and
// in the COL layout (K-major over rows; the operand contracting over rows).
// A weight quantised this way enters the forward and the data-gradient GEMM
// with the same values.
//
// One workgroup of 4 waves owns a 128 x 128 region (4 x 4 squares).  Thread
// t takes row t/2 and the 64 columns of half t%2 (two squares' row segments,
// eight 16-byte loads); the 32 rows of a square are one wave's lanes of one
// parity, so a square's maximum is a 5-step lane exchange.  Codes go out in
// the ROW layout straight from registers (64 contiguous bytes per row) and
// through LDS for the COL layout (each column's 64 bytes from one nibble
// transpose).  SR draws element (r, c) from counter r*cols + c + offset,
// the ROW quantiser's stream, so the codes are those of one quantisation.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

static constexpr int kQ2Threads = 256;
static constexpr int kQ2Rows = 128;
static constexpr int kQ2Cols = 128;
static constexpr int kQ2Stride = 80;  // LDS bytes per staged row of codes (64 + pad)

template <int SR>
__global__ __launch_bounds__(kQ2Threads) void quantize_2d_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint32_t k0,
    uint32_t k1, uint64_t off, uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r,
    uint8_t* __restrict__ codes_c, uint8_t* __restrict__ scales_c) {
    __shared__ __align__(16) uint8_t stage[kQ2Rows * kQ2Stride];
    __shared__ uint8_t tsc[4][4];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int64_t r0 = (int64_t)blockIdx.y * kQ2Rows, c0 = (int64_t)blockIdx.x * kQ2Cols;
    const int r = tid >> 1, h = tid & 1;
    const int64_t gr = r0 + r;
    const bool rok = gr < rows;

    uint4 v[2][4];
    uint32_t amax[2];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t gc = c0 + 64 * h + 32 * t;
        const bool ok = rok && gc < cols;  // cols % 32 == 0: squares wholly in or out
#pragma unroll
        for (int q = 0; q < 4; ++q)
            v[t][q] = ok ? *(const uint4*)(x + gr * ld + gc + 8 * q) : make_uint4(0u, 0u, 0u, 0u);
        u16x2_t m = __builtin_bit_cast(u16x2_t, v[t][0].x & 0x7FFF7FFFu);
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t a = v[t][q].x, b = v[t][q].y, c = v[t][q].z, d = v[t][q].w;
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, a & 0x7FFF7FFFu));
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, b & 0x7FFF7FFFu));
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, c & 0x7FFF7FFFu));
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, d & 0x7FFF7FFFu));
        }
        amax[t] = ((uint32_t)max(m.x, m.y)) << 16;
    }
    // the square's maximum: the 32 lanes of this wave with this parity
#pragma unroll
    for (int t = 0; t < 2; ++t)
#pragma unroll
        for (int msk = 2; msk < 64; msk <<= 1)
            amax[t] = max(amax[t], (uint32_t)__shfl_xor((int)amax[t], msk, 64));

    uint32_t byte[2];
    uint32_t cw[2][4];
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const bool nf = amax[t] >= 0x7F800000u;
        byte[t] = nf ? 0xFFu : e8m0_from_amax(amax[t]);
        const float sc = e8m0_scale_f32(nf ? 0u : byte[t]);
        const int64_t gc = c0 + 64 * h + 32 * t;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const uint32_t w0 = v[t][q].x, w1 = v[t][q].y, w2 = v[t][q].z, w3 = v[t][q].w;
            uint32_t packed = 0;
            if (!SR) {
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w0), sc, 0);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w1), sc, 1);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w2), sc, 2);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w3), sc, 3);
            } else {
                const uint64_t p0 = (uint64_t)gr * (uint64_t)cols + (uint64_t)(gc + 8 * q) + off;
                uint32_t wr[4];
                sr_words8(p0, k0, k1, wr);
                const float xf[8] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1),
                                     bf16_lo(w2), bf16_hi(w2), bf16_lo(w3), bf16_hi(w3)};
                packed = sr_pack8(xf, sc, wr);
            }
            cw[t][q] = nf ? 0u : packed;
        }
        if (rok && gc < cols) {
            *(uint4*)(codes_r + gr * (cols / 2) + gc / 2) =
                make_uint4(cw[t][0], cw[t][1], cw[t][2], cw[t][3]);
            scales_r[gr * (cols / 32) + gc / 32] = (uint8_t)byte[t];
        }
        *(uint4*)(stage + r * kQ2Stride + 32 * h + 16 * t) =
            make_uint4(cw[t][0], cw[t][1], cw[t][2], cw[t][3]);
        if (lane < 2) tsc[wave][2 * h + t] = (uint8_t)byte[t];
    }
    __syncthreads();

    // COL layout: thread -> column c of the region, rows of half `hr`
    // (two squares); byte k of a square's 16 holds rows 2k (low nibble) and
    // 2k + 1 (high nibble) of the column
    const int c = tid & 127, hr = tid >> 7;
    const int64_t gcc = c0 + c;
    if (gcc < cols) {
        const int sh = (c & 1) * 4, bc = c >> 1;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int rb = 2 * hr + s;
            const int64_t grr = r0 + 32 * rb;
            if (grr < rows) {  // rows % 32 == 0: the square's 32 rows are all in
                uint32_t wv[4];
#pragma unroll
                for (int k = 0; k < 4; ++k) {
                    uint32_t w = 0;
#pragma unroll
                    for (int b = 0; b < 4; ++b) {
                        const int rr = 32 * rb + 8 * k + 2 * b;
                        const uint32_t lo = (stage[rr * kQ2Stride + bc] >> sh) & 0xFu;
                        const uint32_t hi = (stage[(rr + 1) * kQ2Stride + bc] >> sh) & 0xFu;
                        w |= (lo | (hi << 4)) << (8 * b);
                    }
                    wv[k] = w;
                }
                *(uint4*)(codes_c + gcc * (rows / 2) + grr / 2) = make_uint4(wv[0], wv[1], wv[2], wv[3]);
                scales_c[gcc * (rows / 32) + grr / 32] = tsc[rb][c >> 5];
            }
        }
    }
}

hipError_t launch_quantize_2d(const void* x, int64_t rows, int64_t cols, int64_t ld, bool sr,
                              uint64_t seed, uint64_t off, uint8_t* codes_r, uint8_t* scales_r,
                              uint8_t* codes_c, uint8_t* scales_c, hipStream_t s) {
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const dim3 grid((unsigned)((cols + kQ2Cols - 1) / kQ2Cols),
                    (unsigned)((rows + kQ2Rows - 1) / kQ2Rows));
    if (sr)
        quantize_2d_kernel<1><<<grid, kQ2Threads, 0, s>>>((const uint16_t*)x, rows, cols, ld, k0, k1,
                                                         off, codes_r, scales_r, codes_c, scales_c);
    else
        quantize_2d_kernel<0><<<grid, kQ2Threads, 0, s>>>((const uint16_t*)x, rows, cols, ld, k0, k1,
                                                         off, codes_r, scales_r, codes_c, scales_c);
    return hipGetLastError();
}

}  // namespace fp4q
