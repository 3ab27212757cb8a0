// Two-dimensional block scaling: one E8M0 scale per TILE x TILE square of a
// bf16 matrix (the recipe of the outlier-dynamics page, sec. 4.1, scales its
// backward operands in 2D blocks; its configuration names 16 x 16 backward
// blocks).  TILE = 32 is MXFP4's 32-element block in both directions, the
// granularity at which the gfx950 scaled MFMA takes scales along K, so the
// one set of codes is written twice: in the ROW layout (blocks along columns;
// the operand of a GEMM contracting over columns) and in the COL layout
// (K-major over rows; the operand contracting over rows).  A weight quantised
// this way enters the forward and the data-gradient GEMM with the same
// values.  TILE = 16 gives the page's 16 x 16 squares in the same two
// layouts with scales per 16 elements: a quantise/dequantise form (the
// hardware GEMM takes one scale per 32 elements).
//
// One workgroup of 4 waves owns a 128 x 128 region.  Thread t takes row t/2
// and the 64 columns of half t%2 (two 32-wide or four 16-wide squares' row
// segments, eight 16-byte loads); the rows of a square are lanes of one
// parity within one wave, so a square's maximum is a 5-step (TILE 32) or
// 4-step (TILE 16) lane exchange.  Codes go out in the ROW layout straight
// from registers (32 contiguous bytes per row) and through LDS for the COL
// layout (each column's 16 bytes per 32 rows from one nibble transpose).  SR
// draws element (r, c) from counter r*cols + c + offset, the ROW
// quantiser's stream, so the codes are those of one quantisation.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

static constexpr int kQ2Threads = 256;
static constexpr int kQ2Rows = 128;
static constexpr int kQ2Cols = 128;
static constexpr int kQ2Stride = 80;  // LDS bytes per staged row of codes (64 + pad)

template <int SR, int TILE>
__global__ __launch_bounds__(kQ2Threads) void quantize_2d_kernel(
    const uint16_t* __restrict__ x, int64_t rows, int64_t cols, int64_t ld, uint32_t k0,
    uint32_t k1, uint64_t off, uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r,
    uint8_t* __restrict__ codes_c, uint8_t* __restrict__ scales_c) {
    static_assert(TILE == 16 || TILE == 32, "16 x 16 or 32 x 32 squares");
    constexpr int SQ = 64 / TILE;   // squares in a thread's 64 columns
    constexpr int QPS = TILE / 8;   // 16-byte loads per square row segment
    constexpr int NT = 128 / TILE;  // squares per region side
    __shared__ __align__(16) uint8_t stage[kQ2Rows * kQ2Stride];
    __shared__ uint8_t tsc[NT][NT];
    const int tid = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * kQ2Rows, c0 = (int64_t)blockIdx.x * kQ2Cols;
    const int r = tid >> 1, h = tid & 1;
    const int64_t gr = r0 + r;
    const bool rok = gr < rows;

    uint4 v[8];
    uint32_t amax[SQ];
#pragma unroll
    for (int sq = 0; sq < SQ; ++sq) {
        const int64_t gc = c0 + 64 * h + TILE * sq;
        const bool ok = rok && gc < cols;  // cols % 32 == 0: squares wholly in or out
#pragma unroll
        for (int q = 0; q < QPS; ++q)
            v[sq * QPS + q] =
                ok ? *(const uint4*)(x + gr * ld + gc + 8 * q) : make_uint4(0u, 0u, 0u, 0u);
        u16x2_t m = __builtin_bit_cast(u16x2_t, v[sq * QPS].x & 0x7FFF7FFFu);
#pragma unroll
        for (int q = 0; q < QPS; ++q) {
            const uint4 w = v[sq * QPS + q];
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w.x & 0x7FFF7FFFu));
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w.y & 0x7FFF7FFFu));
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w.z & 0x7FFF7FFFu));
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, w.w & 0x7FFF7FFFu));
        }
        amax[sq] = ((uint32_t)max(m.x, m.y)) << 16;
    }
    // the square's maximum: the TILE lanes of this wave with this parity whose
    // rows lie in the square (lane = 2 (row % 32) + parity)
#pragma unroll
    for (int sq = 0; sq < SQ; ++sq)
#pragma unroll
        for (int msk = 2; msk < 2 * TILE; msk <<= 1)
            amax[sq] = max(amax[sq], (uint32_t)__shfl_xor((int)amax[sq], msk, 64));

    uint32_t cw[8];
#pragma unroll
    for (int sq = 0; sq < SQ; ++sq) {
        const bool nf = amax[sq] >= 0x7F800000u;
        const uint32_t byte = nf ? 0xFFu : e8m0_from_amax(amax[sq]);
        const float sc = e8m0_scale_f32(nf ? 0u : byte);
        const int64_t gc = c0 + 64 * h + TILE * sq;
#pragma unroll
        for (int q = 0; q < QPS; ++q) {
            const uint4 w = v[sq * QPS + q];
            const uint32_t w0 = w.x, w1 = w.y, w2 = w.z, w3 = w.w;
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
            cw[sq * QPS + q] = nf ? 0u : packed;
        }
        if (rok && gc < cols) scales_r[gr * (cols / TILE) + gc / TILE] = (uint8_t)byte;
        // one lane per square row-block writes the region's scale table
        if ((r % TILE) == 0) tsc[r / TILE][(64 * h) / TILE + sq] = (uint8_t)byte;
    }
#pragma unroll
    for (int t = 0; t < 2; ++t) {
        const int64_t gc = c0 + 64 * h + 32 * t;
        const uint4 o = make_uint4(cw[4 * t], cw[4 * t + 1], cw[4 * t + 2], cw[4 * t + 3]);
        if (rok && gc < cols) *(uint4*)(codes_r + gr * (cols / 2) + gc / 2) = o;
        *(uint4*)(stage + r * kQ2Stride + 32 * h + 16 * t) = o;
    }
    __syncthreads();

    // COL layout: thread -> column c of the region, rows of half `hr`
    // (two 32-row spans); byte k of a span's 16 holds rows 2k (low nibble)
    // and 2k + 1 (high nibble) of the column
    const int c = tid & 127, hr = tid >> 7;
    const int64_t gcc = c0 + c;
    if (gcc < cols) {
        const int sh = (c & 1) * 4, bc = c >> 1;
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int rb = 2 * hr + s;
            const int64_t grr = r0 + 32 * rb;
            if (grr < rows) {  // rows % 32 == 0: the span's 32 rows are all in
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
#pragma unroll
                for (int u = 0; u < 32 / TILE; ++u)
                    scales_c[gcc * (rows / TILE) + grr / TILE + u] =
                        tsc[(32 * rb) / TILE + u][c / TILE];
            }
        }
    }
}

hipError_t launch_quantize_2d(const void* x, int64_t rows, int64_t cols, int64_t ld, int tile,
                              bool sr, uint64_t seed, uint64_t off, uint8_t* codes_r,
                              uint8_t* scales_r, uint8_t* codes_c, uint8_t* scales_c,
                              hipStream_t s) {
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const dim3 grid((unsigned)((cols + kQ2Cols - 1) / kQ2Cols),
                    (unsigned)((rows + kQ2Rows - 1) / kQ2Rows));
    const uint16_t* xb = (const uint16_t*)x;
#define FP4Q_Q2D(SR_, T_)                                                                   \
    FP4Q_LAUNCH((quantize_2d_kernel<SR_, T_>), grid, kQ2Threads, 0, s, xb, rows, cols, ld, k0, k1, off,  \
                                                          codes_r, scales_r, codes_c, scales_c)
    if (tile == 16) {
        if (sr) FP4Q_Q2D(1, 16); else FP4Q_Q2D(0, 16);
    } else {
        if (sr) FP4Q_Q2D(1, 32); else FP4Q_Q2D(0, 32);
    }
#undef FP4Q_Q2D
    return hipGetLastError();
}

}  // namespace fp4q
