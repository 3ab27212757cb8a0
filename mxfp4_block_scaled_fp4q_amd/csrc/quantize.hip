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
//    Each lane owns 8 (bf16) or 4 (fp32) adjacent columns and walks a block of
//    rows with coalesced 16-byte row loads, so the column amax needs no
//    cross-lane traffic and no LDS; it then packs row pairs of one column into
//    bytes and writes each column's block of codes as one 8/16-byte store.
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
            const float inv = e8m0_inv_scale_f32(byte);
            const uint32_t r = rowi[u];
            const uint32_t cc = (valid ? g : 0u) - r * cpr.d;
            const uint64_t p0 = (uint64_t)r * (uint64_t)cols + (uint64_t)cc * 8u + rng_off;
            uint32_t rnd[8];
            sr_bits8(p0, k0, k1, rnd);
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                float xf;
                if (IN_BF16)
                    xf = (j & 1) ? bf16_hi(w[u][j >> 1]) : bf16_lo(w[u][j >> 1]);
                else
                    xf = as_f32(w[u][j]);
                packed |= sr_code(xf, inv, rnd[j]) << (4 * j);
            }
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
// One lane: CPT adjacent columns (16 bytes of a row) x one block of rows,
// processed in sub-blocks of SUB rows held in registers.  Blocks larger than
// SUB take two passes over the rows (amax, then quantise); the second pass
// re-reads rows the first just touched.
template <int IN_BF16, int BLOCK, int SR>
__global__ __launch_bounds__(kThreads) void quantize_col_kernel(
    const void* __restrict__ xv, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint32_t k0, uint32_t k1,
    uint64_t rng_off, int64_t ncg, int64_t nrb, int rb_per_wave) {
    constexpr int CPT = IN_BF16 ? 8 : 4;   // columns per lane
    constexpr int SUB = BLOCK < 32 ? BLOCK : 32;
    constexpr int NSUB = BLOCK / SUB;
    const int lane = threadIdx.x & 63;
    const int64_t cg = (int64_t)blockIdx.x * 64 + lane;
    const int64_t rb0 = ((int64_t)blockIdx.y * (kThreads / 64) + (threadIdx.x >> 6)) * rb_per_wave;
    if (cg >= ncg) return;
    const int64_t c0 = cg * CPT;
    const bool full = (c0 + CPT) <= cols;
    const int64_t half_rows = rows / 2;

    auto load_row = [&](int64_t r, uint32_t (&v)[4]) {
        if (full) {
            const uint4 t = IN_BF16 ? *(const uint4*)((const uint16_t*)xv + r * ld + c0)
                                    : *(const uint4*)((const float*)xv + r * ld + c0);
            v[0] = t.x;
            v[1] = t.y;
            v[2] = t.z;
            v[3] = t.w;
        } else {
            if (IN_BF16) {
                const uint16_t* x = (const uint16_t*)xv + r * ld;
                uint32_t e[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) e[j] = (c0 + j < cols) ? x[c0 + j] : 0u;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = e[2 * j] | (e[2 * j + 1] << 16);
            } else {
                const uint32_t* x = (const uint32_t*)xv + r * ld;
#pragma unroll
                for (int j = 0; j < 4; ++j) v[j] = (c0 + j < cols) ? x[c0 + j] : 0u;
            }
        }
    };
    // fp32 bits of column j of a loaded row
    auto col_bits = [&](const uint32_t (&v)[4], int j) -> uint32_t {
        if (IN_BF16) return (j & 1) ? (v[j >> 1] & 0xFFFF0000u) : (v[j >> 1] << 16);
        return v[j];
    };

    for (int it = 0; it < rb_per_wave; ++it) {
        const int64_t rb = rb0 + it;
        if (rb >= nrb) break;
        const int64_t r0 = rb * BLOCK;
        uint32_t amax[CPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) amax[j] = 0;
        uint32_t v[SUB][4];
        if (NSUB > 1) {
            for (int sb = 0; sb < NSUB; ++sb) {
#pragma unroll
                for (int i = 0; i < SUB; ++i) load_row(r0 + sb * SUB + i, v[i]);
#pragma unroll
                for (int i = 0; i < SUB; ++i)
#pragma unroll
                    for (int j = 0; j < CPT; ++j)
                        amax[j] = max(amax[j], col_bits(v[i], j) & 0x7FFFFFFFu);
            }
        }
        for (int sb = 0; sb < NSUB; ++sb) {
            const int64_t rs = r0 + sb * SUB;
#pragma unroll
            for (int i = 0; i < SUB; ++i) load_row(rs + i, v[i]);
            if (NSUB == 1) {
#pragma unroll
                for (int i = 0; i < SUB; ++i)
#pragma unroll
                    for (int j = 0; j < CPT; ++j)
                        amax[j] = max(amax[j], col_bits(v[i], j) & 0x7FFFFFFFu);
            }
            uint32_t out[CPT][SUB / 8];
#pragma unroll
            for (int j = 0; j < CPT; ++j)
#pragma unroll
                for (int q = 0; q < SUB / 8; ++q) out[j][q] = 0;
            if (!SR) {
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const bool nf = amax[j] >= 0x7F800000u;
                    const float sc = e8m0_scale_f32(nf ? 0xFFu : e8m0_from_amax(amax[j]));
#pragma unroll
                    for (int p = 0; p < SUB / 2; ++p) {
                        uint32_t& dst = out[j][p / 4];
                        if (IN_BF16) {
                            const uint32_t a = col_bits(v[2 * p], j) >> 16;
                            const uint32_t b = col_bits(v[2 * p + 1], j) & 0xFFFF0000u;
                            const bf16x2_t pr = __builtin_bit_cast(bf16x2_t, a | b);
                            switch (p & 3) {
                                case 0: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(dst, pr, sc, 0); break;
                                case 1: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(dst, pr, sc, 1); break;
                                case 2: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(dst, pr, sc, 2); break;
                                default: dst = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(dst, pr, sc, 3); break;
                            }
                        } else {
                            const float a = as_f32(col_bits(v[2 * p], j));
                            const float b = as_f32(col_bits(v[2 * p + 1], j));
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
                float inv[CPT];
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const bool nf = amax[j] >= 0x7F800000u;
                    inv[j] = e8m0_inv_scale_f32(nf ? 0u : e8m0_from_amax(amax[j]));
                }
#pragma unroll
                for (int i = 0; i < SUB; ++i) {
                    uint32_t rnd[8];
                    const uint64_t p0 = (uint64_t)(rs + i) * (uint64_t)cols + (uint64_t)c0 + rng_off;
                    sr_bits8(p0, k0, k1, rnd);
#pragma unroll
                    for (int j = 0; j < CPT; ++j) {
                        const uint32_t code = sr_code(as_f32(col_bits(v[i], j)), inv[j], rnd[j]);
                        out[j][i / 8] |= code << (4 * (i & 7));
                    }
                }
            }
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                if (c0 + j >= cols) break;
                const bool nf = amax[j] >= 0x7F800000u;
                uint8_t* dst = codes + (c0 + j) * half_rows + rs / 2;
                if (SUB == 32) {
                    uint4 t;
                    t.x = nf ? 0u : out[j][0];
                    t.y = nf ? 0u : out[j][1 % (SUB / 8)];
                    t.z = nf ? 0u : out[j][2 % (SUB / 8)];
                    t.w = nf ? 0u : out[j][3 % (SUB / 8)];
                    *(uint4*)dst = t;
                } else {
                    uint2 t;
                    t.x = nf ? 0u : out[j][0];
                    t.y = nf ? 0u : out[j][1 % (SUB / 8)];
                    *(uint2*)dst = t;
                }
            }
        }
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            if (c0 + j >= cols) break;
            const bool nf = amax[j] >= 0x7F800000u;
            scales[(c0 + j) * nrb + rb] = (uint8_t)(nf ? 0xFFu : e8m0_from_amax(amax[j]));
        }
    }
}

template <int IN_BF16, int SR>
static hipError_t col_dispatch(int block, dim3 grid, hipStream_t s, const void* x, int64_t rows,
                               int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                               uint32_t k0, uint32_t k1, uint64_t off, int64_t ncg, int64_t nrb,
                               int rbw) {
    switch (block) {
        case 16:
            quantize_col_kernel<IN_BF16, 16, SR><<<grid, kThreads, 0, s>>>(
                x, rows, cols, ld, codes, scales, k0, k1, off, ncg, nrb, rbw);
            break;
        case 32:
            quantize_col_kernel<IN_BF16, 32, SR><<<grid, kThreads, 0, s>>>(
                x, rows, cols, ld, codes, scales, k0, k1, off, ncg, nrb, rbw);
            break;
        case 64:
            quantize_col_kernel<IN_BF16, 64, SR><<<grid, kThreads, 0, s>>>(
                x, rows, cols, ld, codes, scales, k0, k1, off, ncg, nrb, rbw);
            break;
        default:
            quantize_col_kernel<IN_BF16, 128, SR><<<grid, kThreads, 0, s>>>(
                x, rows, cols, ld, codes, scales, k0, k1, off, ncg, nrb, rbw);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_quantize_col(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                               int block, bool sr, uint64_t seed, uint64_t off, uint8_t* codes,
                               uint8_t* scales, hipStream_t s) {
    const int cpt = dtype == BF16 ? 8 : 4;
    const int64_t ncg = (cols + cpt - 1) / cpt;
    const int64_t nrb = rows / block;
    // Enough waves to fill the chip (a few per SIMD), then more row blocks per
    // wave so each lane writes longer runs of every code row.
    const int64_t col_wgs = (ncg + 63) / 64;
    int rbw = 1;
    while (rbw < 8 && col_wgs * ((nrb + 4 * rbw * 2 - 1) / (4 * rbw * 2)) * 4 >= 8192) rbw *= 2;
    const int64_t wgs_y = (nrb + 4 * rbw - 1) / (4 * rbw);
    dim3 grid((unsigned)col_wgs, (unsigned)wgs_y);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    if (dtype == BF16)
        return sr ? col_dispatch<1, 1>(block, grid, s, x, rows, cols, ld, codes, scales, k0, k1,
                                       off, ncg, nrb, rbw)
                  : col_dispatch<1, 0>(block, grid, s, x, rows, cols, ld, codes, scales, k0, k1,
                                       off, ncg, nrb, rbw);
    return sr ? col_dispatch<0, 1>(block, grid, s, x, rows, cols, ld, codes, scales, k0, k1, off,
                                   ncg, nrb, rbw)
              : col_dispatch<0, 0>(block, grid, s, x, rows, cols, ld, codes, scales, k0, k1, off,
                                   ncg, nrb, rbw);
}

}  // namespace fp4q
