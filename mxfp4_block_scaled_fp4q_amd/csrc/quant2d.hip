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
// One workgroup of 4 waves owns a 128 x 128 region, wave w its 32-row
// block w.  Lane l takes the 16-byte chunk l % 16 of rows 32w + 4q + l / 16
// (q = 0..7): each load instruction reads four whole 256-byte row segments
// of the region.  A square's maximum is the lanes' own maxima combined over
// the chunks of its columns and the four row phases (four lane exchanges,
// three for TILE 16, whose thread rows hold two squares).  Codes go out in
// the ROW layout straight from registers (4 bytes per lane, 64 contiguous
// bytes per row) and through LDS for the COL layout (each column's 16 bytes
// per 32 rows from one nibble transpose).  SR
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
    constexpr int NT = 128 / TILE;  // squares per region side
    __shared__ __align__(16) uint8_t stage[kQ2Rows * kQ2Stride];
    __shared__ uint8_t tsc[NT][NT];
    const int tid = threadIdx.x;
    // Workgroups are dealt to the eight XCDs in turn; remap so that each XCD
    // takes a contiguous run of regions in row-major order: the two 64-byte
    // halves of a row's code line (adjacent regions), most rows' scale lines
    // and, where a run holds whole pairs of region rows, the halves of a
    // column's code line then meet in one L2 and leave it whole (W 2048 x
    // 5632: 15.5 MB written for 11.6 MB of output with a 2D grid before).
    uint32_t reg = blockIdx.x;
    {
        const uint32_t full = (gridDim.x / 8) * 8;
        if (reg < full) reg = (reg % 8) * (full / 8) + reg / 8;
    }
    const uint32_t gx = (uint32_t)((cols + kQ2Cols - 1) / kQ2Cols);
    const uint32_t ry = reg / gx, rx = reg - ry * gx;
    const int64_t r0 = (int64_t)ry * kQ2Rows, c0 = (int64_t)rx * kQ2Cols;
    // Wave w takes the region's rows 32w .. 32w+31 (one 32-row block); lane
    // l takes the 16-byte chunk l % 16 (columns 8 (l % 16) .. +7) of rows
    // 32w + 4q + l / 16, q = 0..7, so that each load instruction reads four
    // whole 256-byte row segments.  A square's maximum is the lanes' own
    // maxima combined over the chunks of its columns (lane bits 0..1 for
    // TILE 32, bit 0 for TILE 16) and the four row phases (bits 4, 5); with
    // TILE 16 the rows of q < 4 and q >= 4 are two squares.
    const int lane = tid & 63, w = tid >> 6;
    const int ch = lane & 15, ph = lane >> 4;
    const int64_t gc = c0 + 8 * ch;
    const bool blk = r0 + 32 * w < rows && gc < cols;  // rows, cols % 32 == 0
    constexpr int HALVES = TILE == 16 ? 2 : 1;  // squares down a thread's rows

    uint4 v[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int64_t gr = r0 + 32 * w + 4 * q + ph;
        v[q] = blk ? *(const uint4*)(x + gr * ld + gc) : make_uint4(0u, 0u, 0u, 0u);
    }
    uint32_t amax[HALVES];
#pragma unroll
    for (int hv = 0; hv < HALVES; ++hv) {
        u16x2_t m = __builtin_bit_cast(u16x2_t, 0u);
#pragma unroll
        for (int q = hv * (8 / HALVES); q < (hv + 1) * (8 / HALVES); ++q) {
            const uint4 t = v[q];
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, t.x & 0x7FFF7FFFu));
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, t.y & 0x7FFF7FFFu));
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, t.z & 0x7FFF7FFFu));
            m = __builtin_elementwise_max(m, __builtin_bit_cast(u16x2_t, t.w & 0x7FFF7FFFu));
        }
        uint32_t a = ((uint32_t)max(m.x, m.y)) << 16;
        a = max(a, (uint32_t)__shfl_xor((int)a, 1, 64));
        if (TILE == 32) a = max(a, (uint32_t)__shfl_xor((int)a, 2, 64));
        a = max(a, (uint32_t)__shfl_xor((int)a, 16, 64));
        a = max(a, (uint32_t)__shfl_xor((int)a, 32, 64));
        amax[hv] = a;
    }

    uint32_t cw[8];
    uint32_t bytes[HALVES];
#pragma unroll
    for (int hv = 0; hv < HALVES; ++hv) {
        const bool nf = amax[hv] >= 0x7F800000u;
        const uint32_t byte = nf ? 0xFFu : e8m0_from_amax(amax[hv]);
        const float sc = e8m0_scale_f32(nf ? 0u : byte);
        bytes[hv] = byte;
#pragma unroll
        for (int q = hv * (8 / HALVES); q < (hv + 1) * (8 / HALVES); ++q) {
            const uint4 t = v[q];
            const uint32_t w0 = t.x, w1 = t.y, w2 = t.z, w3 = t.w;
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
                const int64_t gr = r0 + 32 * w + 4 * q + ph;
                const uint64_t p0 = (uint64_t)gr * (uint64_t)cols + (uint64_t)gc + off;
                uint32_t wr[4];
                sr_words8(p0, k0, k1, wr);
                const float xf[8] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1),
                                     bf16_lo(w2), bf16_hi(w2), bf16_lo(w3), bf16_hi(w3)};
                packed = sr_pack8(xf, sc, wr);
            }
            cw[q] = nf ? 0u : packed;
        }
    }
    // ROW codes: 4 bytes per row from each lane (a 64-byte row segment per 16
    // lanes); ROW scales: one byte per row and square, from the square's
    // first chunk; the staged codes feed the COL layout below
#pragma unroll
    for (int q = 0; q < 8; ++q) {
        const int rl = 32 * w + 4 * q + ph;
        const int64_t gr = r0 + rl;
        if (blk) {
            *(uint32_t*)(codes_r + gr * (cols / 2) + gc / 2) = cw[q];
            if ((ch % (TILE / 8)) == 0)
                scales_r[gr * (cols / TILE) + gc / TILE] = (uint8_t)bytes[q / (8 / HALVES)];
        }
        *(uint32_t*)(stage + rl * kQ2Stride + 4 * ch) = cw[q];
    }
    if (ph == 0 && (ch % (TILE / 8)) == 0) {
#pragma unroll
        for (int hv = 0; hv < HALVES; ++hv)
            tsc[(32 * w) / TILE + hv][(8 * ch) / TILE] = (uint8_t)bytes[hv];
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
    const int64_t regions = ((cols + kQ2Cols - 1) / kQ2Cols) * ((rows + kQ2Rows - 1) / kQ2Rows);
    if (regions >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)regions);
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
