// Fused MXFP4 quantizer: block amax -> E8M0 scale -> scale, round onto E2M1
// (RNE or stochastic) -> two nibbles per byte.
//
// Q(x) = s * round(x / s) with a power-of-two scale shared by each block of
// 16..128 elements (MXFP4 tutorial page, sec. 2.1 and 4.1); E2M1 elements on
// [-6, 6] (outlier-dynamics page, sec. 1.1; MSRA FP4-training summary page,
// sec. 一); 8-bit exponent-only scale (low-precision overview page, sec. 1.1);
// stochastic rounding floor + (rand < frac) (same page, sec. 3.2) with a
// counter-based Philox4x32-10 stream indexed by the element's logical position.
//
// Two kernels, both HBM-streaming:
//  * quantize_row_kernel: blocks along the contiguous dim.  Each lane owns 8
//    consecutive elements (one 16-byte load for bf16, two for fp32); the
//    block/8 lanes of a block reduce their amax with DPP inside a 16-lane row;
//    RNE uses the gfx950 scaled FP4 conversion (x / 2^e, nearest-even,
//    saturating), which matches the E2M1 rounding rule bit for bit; each lane
//    writes one 32-bit word of codes, the block's first lane its scale byte.
//  * quantize_col_kernel: blocks down the strided dim (K-major output of x^T).
//    A workgroup owns one block of rows x 512 (bf16) / 256 (fp32) columns;
//    each wave reads a quarter of the block's rows as contiguous 1 KB row
//    segments (8 or 4 columns per lane), the four partial column maxima
//    meet in LDS, and each column's block of codes is staged in LDS and
//    written as one contiguous store.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

static constexpr int kThreads = 256;

// ---------------------------------------------------------------------------
// ROW
// ---------------------------------------------------------------------------
template <int IN_BF16, int BLOCK, int SR, int UNROLL>
__global__ __launch_bounds__(kThreads) void quantize_row_kernel(
    const void* __restrict__ xv, uint32_t total_chunks, FastDiv cpr, int64_t ld, int64_t cols,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint32_t k0, uint32_t k1,
    uint64_t rng_off) {
    constexpr int G = BLOCK / 8;  // lanes per block
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = (blockIdx.x * (kThreads / 64)) + (threadIdx.x >> 6);
    const uint32_t base = wave * 64u * UNROLL;

    uint32_t w[UNROLL][IN_BF16 ? 4 : 8];
    uint32_t gidx[UNROLL];
    uint32_t rowi[UNROLL];
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        uint32_t g = base + (uint32_t)u * 64u + lane;
        gidx[u] = g;
        uint32_t gg = g < total_chunks ? g : 0u;
        uint32_t r = fastdiv(gg, cpr);
        uint32_t cc = gg - r * cpr.d;
        rowi[u] = r;
        if (IN_BF16) {
            const uint16_t* x = (const uint16_t*)xv;
            uint4 v = *(const uint4*)(x + (int64_t)r * ld + (int64_t)cc * 8);
            w[u][0] = v.x;
            w[u][1] = v.y;
            w[u][2] = v.z;
            w[u][3] = v.w;
        } else {
            const float* x = (const float*)xv;
            const uint4* p = (const uint4*)(x + (int64_t)r * ld + (int64_t)cc * 8);
            uint4 v0 = p[0], v1 = p[1];
            w[u][0] = v0.x;
            w[u][1] = v0.y;
            w[u][2] = v0.z;
            w[u][3] = v0.w;
            w[u][4] = v1.x;
            w[u][5] = v1.y;
            w[u][6] = v1.z;
            w[u][7] = v1.w;
        }
    }
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        const uint32_t g = gidx[u];
        const bool valid = g < total_chunks;
        uint32_t amax;
        if (IN_BF16) {
            u16x2_t m0 = __builtin_bit_cast(u16x2_t, w[u][0] & 0x7FFF7FFFu);
            u16x2_t m1 = __builtin_bit_cast(u16x2_t, w[u][1] & 0x7FFF7FFFu);
            u16x2_t m2 = __builtin_bit_cast(u16x2_t, w[u][2] & 0x7FFF7FFFu);
            u16x2_t m3 = __builtin_bit_cast(u16x2_t, w[u][3] & 0x7FFF7FFFu);
            u16x2_t m = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1),
                                                  __builtin_elementwise_max(m2, m3));
            amax = ((uint32_t)max(m.x, m.y)) << 16;
        } else {
            amax = 0;
#pragma unroll
            for (int j = 0; j < 8; ++j) amax = max(amax, w[u][j] & 0x7FFFFFFFu);
        }
        amax = valid ? amax : 0u;
        amax = group_max_u32<G>(amax);
        const bool nonfinite = amax >= 0x7F800000u;
        const uint32_t byte = nonfinite ? 0xFFu : e8m0_from_amax(amax);
        uint32_t packed = 0;
        if (!SR) {
            const float sc = e8m0_scale_f32(byte);
            if (IN_BF16) {
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w[u][0]), sc, 0);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w[u][1]), sc, 1);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w[u][2]), sc, 2);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w[u][3]), sc, 3);
            } else {
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, as_f32(w[u][0]),
                                                                  as_f32(w[u][1]), sc, 0);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, as_f32(w[u][2]),
                                                                  as_f32(w[u][3]), sc, 1);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, as_f32(w[u][4]),
                                                                  as_f32(w[u][5]), sc, 2);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(packed, as_f32(w[u][6]),
                                                                  as_f32(w[u][7]), sc, 3);
            }
        } else {
            const float sc = e8m0_scale_f32(byte);
            const uint32_t r = rowi[u];
            const uint32_t cc = (valid ? g : 0u) - r * cpr.d;
            const uint64_t p0 = (uint64_t)r * (uint64_t)cols + (uint64_t)cc * 8u + rng_off;
            uint32_t wr[4];
            sr_words8(p0, k0, k1, wr);
            float xf[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (IN_BF16)
                    xf[j] = (j & 1) ? bf16_hi(w[u][j >> 1]) : bf16_lo(w[u][j >> 1]);
                else
                    xf[j] = as_f32(w[u][j]);
            }
            packed = sr_pack8(xf, sc, wr);
        }
        if (nonfinite) packed = 0;
        if (valid) {
            ((uint32_t*)codes)[g] = packed;
            if ((lane % G) == 0) scales[g / G] = (uint8_t)byte;
        }
    }
}

template <int IN_BF16, int SR>
static hipError_t row_dispatch(int block, dim3 grid, hipStream_t s, const void* x, uint32_t tc,
                               FastDiv cpr, int64_t ld, int64_t cols, uint8_t* codes,
                               uint8_t* scales, uint32_t k0, uint32_t k1, uint64_t off) {
    constexpr int U = 4;
    switch (block) {
        case 16:
            quantize_row_kernel<IN_BF16, 16, SR, U><<<grid, kThreads, 0, s>>>(
                x, tc, cpr, ld, cols, codes, scales, k0, k1, off);
            break;
        case 32:
            quantize_row_kernel<IN_BF16, 32, SR, U><<<grid, kThreads, 0, s>>>(
                x, tc, cpr, ld, cols, codes, scales, k0, k1, off);
            break;
        case 64:
            quantize_row_kernel<IN_BF16, 64, SR, U><<<grid, kThreads, 0, s>>>(
                x, tc, cpr, ld, cols, codes, scales, k0, k1, off);
            break;
        default:
            quantize_row_kernel<IN_BF16, 128, SR, U><<<grid, kThreads, 0, s>>>(
                x, tc, cpr, ld, cols, codes, scales, k0, k1, off);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_row(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                               int block, bool sr, uint64_t seed, uint64_t off, uint8_t* codes,
                               uint8_t* scales, hipStream_t s) {
    const uint32_t cpr_n = (uint32_t)(cols / 8);
    const uint32_t tc = (uint32_t)(rows * (int64_t)cpr_n);
    const FastDiv cpr = make_fastdiv(cpr_n);
    const uint32_t per_wg = 64u * 4u * (kThreads / 64);
    dim3 grid((tc + per_wg - 1) / per_wg);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    if (dtype == BF16)
        return sr ? row_dispatch<1, 1>(block, grid, s, x, tc, cpr, ld, cols, codes, scales, k0,
                                       k1, off)
                  : row_dispatch<1, 0>(block, grid, s, x, tc, cpr, ld, cols, codes, scales, k0,
                                       k1, off);
    return sr ? row_dispatch<0, 1>(block, grid, s, x, tc, cpr, ld, cols, codes, scales, k0, k1,
                                   off)
              : row_dispatch<0, 0>(block, grid, s, x, tc, cpr, ld, cols, codes, scales, k0, k1,
                                   off);
}

// ---------------------------------------------------------------------------
// COL
// ---------------------------------------------------------------------------
// One workgroup: one block of BLOCK rows x 64*CPT columns (512 bf16 / 256
// fp32).  Wave w owns rows [w*RPW, (w+1)*RPW) of the block (RPW = BLOCK/4),
// lane l owns columns [l*CPT, (l+1)*CPT): every row load of a wave is one
// contiguous 1 KB segment.  Column maxima of the four row slices meet in
// LDS; each lane then quantises its RPW rows of its CPT columns into
// RPW/2 code bytes per column, staged in LDS so that each column's block of
// codes leaves as one contiguous 8/16/32/64-byte store.
template <int IN_BF16, int BLOCK, int SR>
__global__ __launch_bounds__(kThreads) void quantize_col_kernel(
    const void* __restrict__ xv, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint32_t k0, uint32_t k1,
    uint64_t rng_off, int64_t nrb, int64_t n_cchunks) {
    constexpr int CPT = IN_BF16 ? 8 : 4;  // columns per lane
    constexpr int COLS = 64 * CPT;        // columns per workgroup
    constexpr int RPW = BLOCK / 4;        // rows per wave
    constexpr int WPC = (RPW + 7) / 8;    // 32-bit code words per column per lane
                                          // (block 16: 4 rows -> the low 16 bits)
    __shared__ uint32_t part[4][COLS];                 // per-wave column maxima
    __shared__ __attribute__((aligned(16))) uint32_t cstage[COLS][BLOCK / 8];  // codes

    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t rb = blockIdx.x / n_cchunks;
    const int64_t cc = blockIdx.x - rb * n_cchunks;
    const int64_t c0 = cc * COLS + lane * CPT;
    const bool lane_ok = c0 < cols;
    const bool full = (c0 + CPT) <= cols;
    const int64_t r0 = rb * BLOCK + wave * RPW;

    uint32_t v[RPW][4];
#pragma unroll
    for (int i = 0; i < RPW; ++i) {
        const int64_t r = r0 + i;
        if (full) {
            const uint4 t = IN_BF16 ? *(const uint4*)((const uint16_t*)xv + r * ld + c0)
                                    : *(const uint4*)((const float*)xv + r * ld + c0);
            v[i][0] = t.x;
            v[i][1] = t.y;
            v[i][2] = t.z;
            v[i][3] = t.w;
        } else if (IN_BF16) {
            const uint16_t* x = (const uint16_t*)xv + r * ld;
            uint32_t e[8];
#pragma unroll
            for (int j = 0; j < 8; ++j) e[j] = (c0 + j < cols) ? x[c0 + j] : 0u;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[i][j] = e[2 * j] | (e[2 * j + 1] << 16);
        } else {
            const uint32_t* x = (const uint32_t*)xv + r * ld;
#pragma unroll
            for (int j = 0; j < 4; ++j) v[i][j] = (c0 + j < cols) ? x[c0 + j] : 0u;
        }
    }
    auto col_bits = [&](int i, int j) -> uint32_t {
        if (IN_BF16) return (j & 1) ? (v[i][j >> 1] & 0xFFFF0000u) : (v[i][j >> 1] << 16);
        return v[i][j];
    };

    // column maxima of this wave's rows, then across the four waves
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < RPW; ++i) m = max(m, col_bits(i, j) & 0x7FFFFFFFu);
        part[wave][lane * CPT + j] = m;
    }
    __syncthreads();
    uint32_t amax[CPT];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
        amax[j] = max(max(part[0][lane * CPT + j], part[1][lane * CPT + j]),
                      max(part[2][lane * CPT + j], part[3][lane * CPT + j]));

    uint32_t out[CPT][WPC];
#pragma unroll
    for (int j = 0; j < CPT; ++j)
#pragma unroll
        for (int q = 0; q < WPC; ++q) out[j][q] = 0;
    if (!SR) {
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const bool nf = amax[j] >= 0x7F800000u;
            const float sc = e8m0_scale_f32(nf ? 0xFFu : e8m0_from_amax(amax[j]));
#pragma unroll
            for (int p = 0; p < RPW / 2; ++p) {
                uint32_t& dst = out[j][p / 4];
                if (IN_BF16) {
                    const uint32_t a = col_bits(2 * p, j) >> 16;
                    const uint32_t b = col_bits(2 * p + 1, j) & 0xFFFF0000u;
                    const bf16x2_t pr = __builtin_bit_cast(bf16x2_t, a | b);
                    switch (p & 3) {
                        case 0: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(dst, pr, sc, 0); break;
                        case 1: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(dst, pr, sc, 1); break;
                        case 2: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(dst, pr, sc, 2); break;
                        default: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(dst, pr, sc, 3); break;
                    }
                } else {
                    const float a = as_f32(col_bits(2 * p, j));
                    const float b = as_f32(col_bits(2 * p + 1, j));
                    switch (p & 3) {
                        case 0: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dst, a, b, sc, 0); break;
                        case 1: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dst, a, b, sc, 1); break;
                        case 2: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dst, a, b, sc, 2); break;
                        default: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(dst, a, b, sc, 3); break;
                    }
                }
            }
        }
    } else {
        float sc[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const bool nf = amax[j] >= 0x7F800000u;
            sc[j] = e8m0_scale_f32(nf ? 0u : e8m0_from_amax(amax[j]));
        }
        // rows i, i+1 of a column form one code byte (byte (i % 8) / 2 of word
        // i / 8); column j's 16-bit lane is half j & 1 of word j / 2 of the
        // row's random words
#pragma unroll
        for (int i = 0; i < RPW; i += 2) {
            uint32_t w0[4], w1[4];
            const uint64_t p0 = (uint64_t)(r0 + i) * (uint64_t)cols + (uint64_t)c0 + rng_off;
            sr_words8(p0, k0, k1, w0);
            sr_words8(p0 + (uint64_t)cols, k0, k1, w1);
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const uint32_t u0 = (w0[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
                const uint32_t u1 = (w1[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
                out[j][i / 8] |= sr_pair(as_f32(col_bits(i, j)), as_f32(col_bits(i + 1, j)), sc[j],
                                         u0 << 16, u1 << 15)
                                 << (8 * ((i & 7) >> 1));
            }
        }
    }
    // stage: column (lane*CPT + j), words [wave*WPC, (wave+1)*WPC) of its block
#pragma unroll
    for (int j = 0; j < CPT; ++j) {
        const bool nf = amax[j] >= 0x7F800000u;
        if (RPW >= 8) {
#pragma unroll
            for (int q = 0; q < WPC; ++q)
                cstage[lane * CPT + j][wave * WPC + q] = nf ? 0u : out[j][q];
        } else {
            ((uint16_t*)cstage[lane * CPT + j])[wave] = (uint16_t)(nf ? 0u : out[j][0]);
        }
    }
    if (wave == 0 && lane_ok) {
#pragma unroll
        for (int j = 0; j < CPT; ++j)
            if (c0 + j < cols)
                scales[(c0 + j) * nrb + rb] =
                    (uint8_t)(amax[j] >= 0x7F800000u ? 0xFFu : e8m0_from_amax(amax[j]));
    }
    __syncthreads();
    // store: thread t writes whole columns' code blocks (BLOCK/2 bytes each)
    const int64_t half_rows = rows / 2;
    constexpr int WORDS = BLOCK / 8;
    for (int col = threadIdx.x; col < COLS; col += kThreads) {
        const int64_t c = cc * COLS + col;
        if (c >= cols) break;
        uint8_t* dst = codes + c * half_rows + rb * (BLOCK / 2);
        const uint32_t* src = cstage[col];
        if (WORDS >= 4) {
#pragma unroll
            for (int q = 0; q < WORDS; q += 4)
                *(uint4*)(dst + 4 * q) = make_uint4(src[q], src[q + 1], src[q + 2], src[q + 3]);
        } else {
            *(uint2*)dst = make_uint2(src[0], src[1 % WORDS]);
        }
    }
}

template <int IN_BF16, int SR>
static hipError_t col_dispatch(int block, dim3 grid, hipStream_t s, const void* x, int64_t rows,
                               int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                               uint32_t k0, uint32_t k1, uint64_t off, int64_t nrb, int64_t ncc) {
    switch (block) {
        case 16:
            quantize_col_kernel<IN_BF16, 16, SR><<<grid, kThreads, 0, s>>>(
                x, rows, cols, ld, codes, scales, k0, k1, off, nrb, ncc);
            break;
        case 32:
            quantize_col_kernel<IN_BF16, 32, SR><<<grid, kThreads, 0, s>>>(
                x, rows, cols, ld, codes, scales, k0, k1, off, nrb, ncc);
            break;
        case 64:
            quantize_col_kernel<IN_BF16, 64, SR><<<grid, kThreads, 0, s>>>(
                x, rows, cols, ld, codes, scales, k0, k1, off, nrb, ncc);
            break;
        default:
            quantize_col_kernel<IN_BF16, 128, SR><<<grid, kThreads, 0, s>>>(
                x, rows, cols, ld, codes, scales, k0, k1, off, nrb, ncc);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_col(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                               int block, bool sr, uint64_t seed, uint64_t off, uint8_t* codes,
                               uint8_t* scales, hipStream_t s) {
    const int64_t cols_per_wg = dtype == BF16 ? 512 : 256;
    const int64_t ncc = (cols + cols_per_wg - 1) / cols_per_wg;
    const int64_t nrb = rows / block;
    dim3 grid((unsigned)(nrb * ncc));
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    if (dtype == BF16)
        return sr ? col_dispatch<1, 1>(block, grid, s, x, rows, cols, ld, codes, scales, k0, k1,
                                       off, nrb, ncc)
                  : col_dispatch<1, 0>(block, grid, s, x, rows, cols, ld, codes, scales, k0, k1,
                                       off, nrb, ncc);
    return sr ? col_dispatch<0, 1>(block, grid, s, x, rows, cols, ld, codes, scales, k0, k1, off,
                                   nrb, ncc)
              : col_dispatch<0, 0>(block, grid, s, x, rows, cols, ld, codes, scales, k0, k1, off,
                                   nrb, ncc);
}

}  // namespace fp4q
