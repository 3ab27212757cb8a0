// Fused MXFP4 quantizer: block amax -> E8M0 scale -> scale, round onto E2M1
// (RNE or stochastic) -> two nibbles per byte.
//
// Q(x) = s * round(x / s) with a power-of-two scale shared by each block of
// 16..128 elements (MXFP4 tutorial page, sec. 2.1 and 4.1); E2M1 elements on
// [-6, 6] (outlier-dynamics page, sec. 1.1; MSRA FP4-training summary page,
// sec. 一); 8-bit exponent-only scale (low-precision overview page, sec. 1.1);
// stochastic rounding (same page, sec. 3.2: up with probability equal to the
// fractional distance) at 16-bit resolution: up iff u + floor(frac * 2^16)
// carries out of 16 bits, u from a counter-based Philox4x32-10 stream indexed
// by the element's logical position.
//
// Two kernels, both HBM-streaming:
//  * quantize_row_kernel: blocks along the contiguous dim.  Each lane owns 8
//    consecutive elements (one 16-byte load for bf16, two for fp32); the
//    block/8 lanes of a block reduce their amax with DPP inside a 16-lane row;
//    RNE uses the gfx950 scaled FP4 conversion (x / 2^e, nearest-even,
//    saturating), which matches the E2M1 rounding rule bit for bit; each lane
//    writes one 32-bit word of codes, the block's first lane its scale byte.
//  * quantize_col_kernel: blocks down the strided dim (K-major output of x^T).
//    A workgroup owns a tile of 128 or 256 rows x 128 (bf16) / 64 (fp32)
//    columns; each lane reads 8 or 16 rows of 16 bytes, the partial column
//    maxima of a block's row groups meet in LDS, and each column's codes are
//    staged in LDS and leave as contiguous segments.  The bf16 form can also
//    write the ROW quantisation of the same tile (one read, both layouts).

#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

static constexpr int kThreads = 256;

// A block's E8M0 byte, conversion scale and code mask from the biased
// exponent t (0..255) of its largest magnitude, with no selects: byte =
// max(t - 2, 0) (floor(log2 amax) - 2, biased), or 0xFF where t = 255 (Inf
// or NaN in the block); sc = 2^(byte - 127) (the scale operand of the scaled
// conversions; fp32 denormals are preserved, so byte 0 gives 2^-127); keep
// is all ones, or zero for an Inf/NaN block (whose codes are zeros).
struct BlockScale {
    uint32_t byte, keep;
    float sc;
};
__device__ __forceinline__ BlockScale block_scale(uint32_t t) {
    const uint32_t n8 = (t + 1u) >> 8;  // 1 iff t == 255
    const uint32_t e = __builtin_elementwise_sub_sat(t, 2u);
    BlockScale r;
    r.byte = e + 2u * n8;
    r.keep = n8 - 1u;
    r.sc = __builtin_amdgcn_ldexpf(0x1p-127f, (int)e);
    return r;
}

// ---------------------------------------------------------------------------
// ROW
// ---------------------------------------------------------------------------
// zmask (optional): one bit per column; set columns are quantised as zeros.
// MASK (compile-time, so that the unmasked kernel holds no mask loads: a mask
// load among the data loads made the compiler wait for each data load before
// issuing the next) says that zmask is given.
template <int IN_BF16, int BLOCK, int SR, int UNROLL, int MASK>
__global__ __launch_bounds__(kThreads) void quantize_row_kernel(
    const void* __restrict__ xv, uint32_t total_chunks, FastDiv cpr, int64_t ld, int64_t cols,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint32_t k0, uint32_t k1,
    uint64_t rng_off, const uint32_t* __restrict__ zmask) {
    constexpr int G = BLOCK / 8;  // lanes per block
    const uint32_t lane = threadIdx.x & 63u;
    const uint32_t wave = (blockIdx.x * (kThreads / 64)) + (threadIdx.x >> 6);
    const uint32_t base = wave * 64u * UNROLL;

    uint32_t w[UNROLL][IN_BF16 ? 4 : 8];
    uint32_t gidx[UNROLL];
    uint32_t rowi[UNROLL];
    // dense rows (ld == cols) without a mask: chunk g starts at element 8 g,
    // and neither rounding needs the row index (the stochastic one's position
    // is 8 g + offset), so no division
    const bool flat = !MASK && ld == cols;
    if (flat) {
        // the input is read once: non-temporal loads (plain ones for the
        // stochastic form, which is bound by its arithmetic), all in flight
        // together (chunks past the end load chunk 0, unused; no branch
        // around a load)
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const uint32_t g = base + (uint32_t)u * 64u + lane;
            gidx[u] = g;
            rowi[u] = 0;
            const uint4* p = (const uint4*)xv + (IN_BF16 ? 1 : 2) * (g < total_chunks ? g : 0u);
            const uint4 v0 = SR ? *p : load_nt(p);
            w[u][0] = v0.x;
            w[u][1] = v0.y;
            w[u][2] = v0.z;
            w[u][3] = v0.w;
            if (!IN_BF16) {
                const uint4 v1 = SR ? p[1] : load_nt(p + 1);
                w[u][4 % (IN_BF16 ? 4 : 8)] = v1.x;
                w[u][5 % (IN_BF16 ? 4 : 8)] = v1.y;
                w[u][6 % (IN_BF16 ? 4 : 8)] = v1.z;
                w[u][7 % (IN_BF16 ? 4 : 8)] = v1.w;
            }
        }
    } else {
#pragma unroll
    for (int u = 0; u < UNROLL; ++u) {
        uint32_t g = base + (uint32_t)u * 64u + lane;
        gidx[u] = g;
        uint32_t gg = g < total_chunks ? g : 0u;
        const uint32_t r = fastdiv(gg, cpr);
        const uint32_t cc = gg - r * cpr.d;
        rowi[u] = r;
        // the input is read once: non-temporal loads, except for the
        // stochastic form, which is bound by its arithmetic and measured
        // faster with plain loads (dY 8192 x 5632 cold: 27.4 against 28.6 us)
        if (IN_BF16) {
            const uint16_t* x = (const uint16_t*)xv;
            const uint4* p = (const uint4*)(x + (int64_t)r * ld + (int64_t)cc * 8);
            uint4 v = SR ? *p : load_nt(p);
            w[u][0] = v.x;
            w[u][1] = v.y;
            w[u][2] = v.z;
            w[u][3] = v.w;
        } else {
            const float* x = (const float*)xv;
            const uint4* p = (const uint4*)(x + (int64_t)r * ld + (int64_t)cc * 8);
            uint4 v0 = SR ? p[0] : load_nt(p), v1 = SR ? p[1] : load_nt(p + 1);
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
    }
    if (MASK) {
        // after every data load is in flight: the chunk's 8 columns are bits
        // 8 (cc % 4) .. +7 of word cc / 4
#pragma unroll
        for (int u = 0; u < UNROLL; ++u) {
            const uint32_t gg = gidx[u] < total_chunks ? gidx[u] : 0u;
            const uint32_t cc = gg - rowi[u] * cpr.d;
            const uint32_t mb = (zmask[cc >> 2] >> ((cc & 3) * 8)) & 0xFFu;
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                if (!((mb >> j) & 1u)) continue;
                if (IN_BF16)
                    w[u][j >> 1] &= (j & 1) ? 0x0000FFFFu : 0xFFFF0000u;
                else
                    w[u][j % (IN_BF16 ? 4 : 8)] = 0u;
            }
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
            // position of the chunk's first element: r * cols + 8 cc = 8 g
            const uint64_t p0 = (uint64_t)(valid ? g : 0u) * 8u + rng_off;
            uint32_t wr[4];
            if ((rng_off & 7) == 0) {
                // (a workgroup-uniform test) the chunk is one Philox counter
                const uint64_t n = p0 >> 3;
                const Philox4 a = philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), 0u, 0u, k0, k1);
#pragma unroll
                for (int k = 0; k < 4; ++k) wr[k] = a.v[k];
            } else {
                sr_words8(p0, k0, k1, wr);
            }
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

template <int IN_BF16, int SR, int MASK>
static hipError_t row_dispatch(int block, dim3 grid, hipStream_t s, const void* x, uint32_t tc,
                               FastDiv cpr, int64_t ld, int64_t cols, uint8_t* codes,
                               uint8_t* scales, uint32_t k0, uint32_t k1, uint64_t off,
                               const uint32_t* zmask) {
    // chunks per lane: 4 for nearest-even (all loads in flight, then a short
    // convert); 2 for the stochastic form, whose long convert (Philox per
    // chunk) otherwise holds each wave's next loads back: dY 8192 x 5632
    // streamed cold 30.5 -> 28.3 us (4 -> 2; 8: 33.1 us, 1: 30.6 us)
    constexpr int U = SR ? 2 : 4;
    switch (block) {
        case 16:
            FP4Q_LAUNCH((quantize_row_kernel<IN_BF16, 16, SR, U, MASK>), grid, kThreads, 0, s,
                x, tc, cpr, ld, cols, codes, scales, k0, k1, off, zmask);
            break;
        case 32:
            FP4Q_LAUNCH((quantize_row_kernel<IN_BF16, 32, SR, U, MASK>), grid, kThreads, 0, s,
                x, tc, cpr, ld, cols, codes, scales, k0, k1, off, zmask);
            break;
        case 64:
            FP4Q_LAUNCH((quantize_row_kernel<IN_BF16, 64, SR, U, MASK>), grid, kThreads, 0, s,
                x, tc, cpr, ld, cols, codes, scales, k0, k1, off, zmask);
            break;
        default:
            FP4Q_LAUNCH((quantize_row_kernel<IN_BF16, 128, SR, U, MASK>), grid, kThreads, 0, s,
                x, tc, cpr, ld, cols, codes, scales, k0, k1, off, zmask);
            break;
    }
    return hipGetLastError();
}

template <int IN_BF16, int SR>
static hipError_t row_dispatch_mask(int block, dim3 grid, hipStream_t s, const void* x,
                                    uint32_t tc, FastDiv cpr, int64_t ld, int64_t cols,
                                    uint8_t* codes, uint8_t* scales, uint32_t k0, uint32_t k1,
                                    uint64_t off, const uint32_t* zmask) {
    return zmask ? row_dispatch<IN_BF16, SR, 1>(block, grid, s, x, tc, cpr, ld, cols, codes,
                                                scales, k0, k1, off, zmask)
                 : row_dispatch<IN_BF16, SR, 0>(block, grid, s, x, tc, cpr, ld, cols, codes,
                                                scales, k0, k1, off, zmask);
}

hipError_t launch_quantize_row(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                               int block, bool sr, uint64_t seed, uint64_t off, uint8_t* codes,
                               uint8_t* scales, hipStream_t s, const uint32_t* zmask) {
    const uint32_t cpr_n = (uint32_t)(cols / 8);
    const uint32_t tc = (uint32_t)(rows * (int64_t)cpr_n);
    const FastDiv cpr = make_fastdiv(cpr_n);
    const uint32_t per_wg = 64u * (sr ? 2u : 4u) * (kThreads / 64);  // U chunks per lane
    dim3 grid((tc + per_wg - 1) / per_wg);
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    if (dtype == BF16)
        return sr ? row_dispatch_mask<1, 1>(block, grid, s, x, tc, cpr, ld, cols, codes, scales, k0,
                                       k1, off, zmask)
                  : row_dispatch_mask<1, 0>(block, grid, s, x, tc, cpr, ld, cols, codes, scales, k0,
                                       k1, off, zmask);
    return sr ? row_dispatch_mask<0, 1>(block, grid, s, x, tc, cpr, ld, cols, codes, scales, k0, k1,
                                   off, zmask)
              : row_dispatch_mask<0, 0>(block, grid, s, x, tc, cpr, ld, cols, codes, scales, k0, k1,
                                   off, zmask);
}

// ---------------------------------------------------------------------------
// COL
// ---------------------------------------------------------------------------
// One workgroup (256 threads) quantises a tile of TR = 16*RPT rows x TC
// columns (TC = 128 bf16 / 64 fp32, 256 bytes of each row; RPT = 16, or 8
// where the stochastic passes need the registers).  Thread (rg, cg) =
// (tid / 16, tid % 16) holds rows rg*RPT .. rg*RPT+RPT-1 of columns
// cg*CPT .. cg*CPT+CPT-1, one 16-byte load per row, so a wave's load covers
// four 256-byte row segments.  Block maxima over the BLOCK/RPT row groups of
// a block meet in LDS.  Each thread turns its RPT rows of a column into RPT/2
// code bytes; they are staged in LDS per column, and the tile's output (each
// column's TR/2 contiguous code bytes, i.e. K-major rows of the transposed
// operand) leaves as one contiguous segment per column (128 or 64 bytes)
// written by consecutive lanes, which is what makes this layout change run
// at streaming speed.
// ALIGNED (cols a multiple of 8, and for the stochastic passes the offset
// too): a lane's columns lie all inside or all outside the matrix, so its
// loads need no per-element edge tests, and every row's positions
// c0 .. c0+CPT-1 lie in one Philox counter, so each row takes one call.
//
// ROW != 0 (bf16 only, cols % BLOCK == 0): the same pass also writes the ROW
// quantisation of the tile (ROW = 1 nearest-even, 2 stochastic with key
// kr0, kr1, 3 stochastic with the column pass's key, so one Philox stream
// serves both): each thread's 8 columns of a row are a quarter/half/... of a
// row block whose BLOCK/8 threads are adjacent lanes of one 16-lane row,
// so the row-block maximum is a DPP reduction.
template <int IN_BF16, int BLOCK, int SR, int ALIGNED, int ROW, int RPT>
__global__ __launch_bounds__(kThreads) void quantize_col_kernel(
    const void* __restrict__ xv, int64_t rows, int64_t cols, int64_t ld,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint32_t k0, uint32_t k1,
    uint64_t rng_off, int64_t nrb, FastDiv n_ctiles,
    uint8_t* __restrict__ codes_r, uint8_t* __restrict__ scales_r, uint32_t kr0, uint32_t kr1,
    const uint32_t* __restrict__ zmask) {
    static_assert(ROW == 0 || IN_BF16, "the fused row pass is for bf16 input");
    static_assert(ROW != 3 || SR, "a shared random stream needs the stochastic column pass");
    constexpr int RG = BLOCK / 8;  // lanes per row block (fused row pass)
    constexpr int CPT = IN_BF16 ? 8 : 4;  // columns per thread
    constexpr int TC = 16 * CPT;          // columns per tile
    constexpr int TR = 16 * RPT;          // rows per tile (RPT rows per thread: 16, or 8
                                          // where the stochastic passes need registers)
    constexpr int NPB = BLOCK / RPT;      // row groups per block
    constexpr int WPT = RPT / 8;          // code words per column per thread
    static_assert(RPT == 8 || RPT == 16, "8 or 16 rows per thread");
    constexpr int BPT = TR / BLOCK;       // blocks per tile (per column)
    constexpr int PITCH = TR / 2 + 16;    // staged code bytes per column (padded)
    constexpr int ES = IN_BF16 ? 2 : 4;   // input element bytes
    static_assert(kThreads == 256, "16 x 16 thread layout");
    __shared__ __attribute__((aligned(16))) uint32_t part[NPB > 1 ? 16 : 1][TC];
    __shared__ __attribute__((aligned(16))) uint8_t cst[TC * PITCH];
    __shared__ uint8_t sst[TC][BPT];

    const int tid = threadIdx.x;
    const int cg = tid & 15, rg = tid >> 4;
    // Workgroups are dealt to the eight XCDs in turn; remap so that each XCD
    // takes a contiguous run of tiles (row-major), whose partial-line writes
    // (row codes and scales, column scales) then meet in that XCD's L2.
    uint32_t tile = blockIdx.x;
    {
        const uint32_t full = (gridDim.x / 8) * 8;
        if (tile < full) tile = (tile % 8) * (full / 8) + tile / 8;
    }

    // Loads of tile t into v: this thread's RPT rows of its CPT columns.
    // ALIGNED (cols % 8 == 0): a lane's columns lie all inside or all outside
    // the matrix, and its RPT rows too (rows are a multiple of the block), so
    // the RPT 16-byte loads are unconditional (all in flight together): a
    // lane outside reads the tile's first rows and columns instead.
    // Otherwise (a lane's columns may straddle the edge): element loads at
    // the edge.
    auto load = [&](uint32_t t, uint32_t (&v)[RPT][4]) {
        const uint32_t trow = fastdiv(t, n_ctiles);
        const uint32_t tcol = t - trow * n_ctiles.d;
        const int64_t r0 = (int64_t)trow * TR;
        const int64_t c0 = (int64_t)tcol * TC + cg * CPT;
        const bool rows_ok = rg * RPT < rows - r0;
        if (ALIGNED) {
            // a workgroup-uniform tile base and 32-bit lane offsets (the host
            // keeps a tile's extent below 2^31 bytes); a lane outside reads
            // rows r0.. of the tile's first columns, which exist
            const bool ok = rows_ok && c0 + CPT <= cols;
            const char* const tb = (const char*)xv + (r0 * ld + (int64_t)tcol * TC) * ES;
            const uint32_t lo =
                ok ? (uint32_t)(rg * RPT) * (uint32_t)(ld * ES) + (uint32_t)(cg * CPT * ES) : 0u;
            const uint32_t rs = (uint32_t)(ld * ES);
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const uint4 u = *(const uint4*)(tb + (lo + i * rs));
                v[i][0] = u.x;
                v[i][1] = u.y;
                v[i][2] = u.z;
                v[i][3] = u.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int64_t r = r0 + rg * RPT + i;
                if (rows_ok && c0 + CPT <= cols) {
                    const uint4 u = IN_BF16 ? *(const uint4*)((const uint16_t*)xv + r * ld + c0)
                                            : *(const uint4*)((const float*)xv + r * ld + c0);
                    v[i][0] = u.x;
                    v[i][1] = u.y;
                    v[i][2] = u.z;
                    v[i][3] = u.w;
                } else if (rows_ok && IN_BF16) {
                    const uint16_t* x = (const uint16_t*)xv + r * ld;
                    uint32_t e[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) e[j] = (c0 + j < cols) ? x[c0 + j] : 0u;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[i][j] = e[2 * j] | (e[2 * j + 1] << 16);
                } else if (rows_ok) {
                    const uint32_t* x = (const uint32_t*)xv + r * ld;
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[i][j] = (c0 + j < cols) ? x[c0 + j] : 0u;
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[i][j] = 0u;
                }
            }
        }
    };

    // Everything after the loads of tile t: scales, codes, LDS staging and
    // the tile's stores.
    auto process = [&](uint32_t t, uint32_t (&v)[RPT][4]) {
        const uint32_t trow = fastdiv(t, n_ctiles);
        const int64_t tcol = t - trow * n_ctiles.d;
        const int64_t r0 = (int64_t)trow * TR;              // first row of the tile
        const int64_t c0 = tcol * TC + cg * CPT;            // first column of this thread
        const int64_t rem = rows - r0;
        const int vrows = rem < TR ? (int)rem : TR;         // a multiple of the block
        const bool rows_ok = rg * RPT < vrows;
        // a whole tile inside the matrix (workgroup-uniform): no per-lane tests
        const bool interior = rem >= TR && (tcol + 1) * TC <= cols;

        // (ALIGNED: a lane outside the matrix holds values read from its first
        // rows; they reach no stored output: blocks in either direction lie
        // wholly inside or wholly outside, and only inside ones are stored)
        if (ROW == 0 && zmask && rows_ok) {
            // one bit per row; set rows are quantised as zeros (the thread's RPT
            // rows start at a multiple of RPT, so their bits lie in one word)
            const int64_t rf = r0 + rg * RPT;
            const uint32_t mb = (zmask[rf >> 5] >> (rf & 31)) & ((1u << RPT) - 1u);
#pragma unroll
            for (int i = 0; i < RPT; ++i)
                if ((mb >> i) & 1u)
#pragma unroll
                    for (int j = 0; j < 4; ++j) v[i][j] = 0u;
        }
        auto col_bits = [&](int i, int j) -> uint32_t {
            if (IN_BF16) return (j & 1) ? (v[i][j >> 1] & 0xFFFF0000u) : (v[i][j >> 1] << 16);
            return v[i][j];
        };
        // scale of the row block holding thread row i: the largest bf16
        // magnitude (16-bit pattern) of the lane's 8 values, then a DPP maximum
        // over the block's RG lanes, whose bits 7.. are the biased exponent
        auto row_scale = [&](int i) -> BlockScale {
            const u16x2_t m0 = __builtin_bit_cast(u16x2_t, v[i][0] & 0x7FFF7FFFu);
            const u16x2_t m1 = __builtin_bit_cast(u16x2_t, v[i][1] & 0x7FFF7FFFu);
            const u16x2_t m2 = __builtin_bit_cast(u16x2_t, v[i][2] & 0x7FFF7FFFu);
            const u16x2_t m3 = __builtin_bit_cast(u16x2_t, v[i][3] & 0x7FFF7FFFu);
            const u16x2_t mm = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1),
                                                         __builtin_elementwise_max(m2, m3));
            const uint32_t ra = group_max_u32<RG>((uint32_t)max(mm.x, mm.y));
            return block_scale(ra >> 7);
        };
        // ROW codes and scales of this thread's row i: a uniform tile base plus
        // a lane offset (32-bit where ALIGNED: the host keeps it below 2^31)
        const int64_t rcodes = cols / 2, rscales = cols / BLOCK;
        uint8_t* const rcb = codes_r + r0 * rcodes + tcol * (TC / 2);
        uint8_t* const rsb = scales_r + r0 * rscales + tcol * (TC / BLOCK);
        // (the lane parts are fixed once and hidden from the optimiser, which
        // would otherwise fold them with the row steps into one multiply per
        // row)
        uint32_t rc_lane = (uint32_t)(rg * RPT) * (uint32_t)rcodes + cg * 4;
        uint32_t rs_lane = (uint32_t)(rg * RPT) * (uint32_t)rscales + (cg * 8) / BLOCK;
        if (ALIGNED && ROW) asm volatile("" : "+v"(rc_lane), "+v"(rs_lane));
        auto rcode_at = [&](int i) -> uint8_t* {
            return ALIGNED ? rcb + (rc_lane + (uint32_t)i * (uint32_t)rcodes)
                           : rcb + ((rg * RPT + i) * rcodes + cg * 4);
        };
        auto rscale_at = [&](int i) -> uint8_t* {
            return ALIGNED ? rsb + (rs_lane + (uint32_t)i * (uint32_t)rscales)
                           : rsb + ((rg * RPT + i) * rscales + (cg * 8) / BLOCK);
        };

        if (ROW == 1) {
            // ROW blocks, nearest-even: every row's codes first, then the stores
            // under one test (the rows' conversions interleave)
            uint32_t rpk[RPT], rby[RPT];
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const BlockScale bs = row_scale(i);
                uint32_t packed = 0;
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, v[i][0]), bs.sc, 0);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, v[i][1]), bs.sc, 1);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, v[i][2]), bs.sc, 2);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, v[i][3]), bs.sc, 3);
                rpk[i] = packed & bs.keep;
                rby[i] = bs.byte;
            }
            if (interior || (rows_ok && c0 < cols)) {
                // (the RG lanes of a block hold the same byte and all store it)
#pragma unroll
                for (int i = 0; i < RPT; ++i) {
                    *(uint32_t*)rcode_at(i) = rpk[i];
                    *rscale_at(i) = (uint8_t)rby[i];
                }
            }
        }
        if (ROW == 2) {
            // ROW blocks, stochastic with their own key: one row at a time
#pragma unroll
            for (int i = 0; i < RPT; ++i) {
                const int64_t r = r0 + rg * RPT + i;
                const BlockScale bs = row_scale(i);
                const uint32_t rbyte = bs.byte;
                const float rsc = bs.sc;
                uint32_t packed;
                {
                    uint32_t wr[4];
                    const uint64_t q0 = (uint64_t)r * (uint64_t)cols + (uint64_t)c0 + rng_off;
                    if (ALIGNED) {
                        const uint64_t n0 = q0 >> 3;
                        const Philox4 a =
                            philox4x32_10((uint32_t)n0, (uint32_t)(n0 >> 32), 0u, 0u, kr0, kr1);
#pragma unroll
                        for (int k = 0; k < 4; ++k) wr[k] = a.v[k];
                    } else {
                        sr_words8(q0, kr0, kr1, wr);
                    }
                    float xf[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j)
                        xf[j] = (j & 1) ? bf16_hi(v[i][j >> 1]) : bf16_lo(v[i][j >> 1]);
                    packed = sr_pack8(xf, rsc, wr);
                }
                packed &= bs.keep;
                if (interior || (rows_ok && c0 < cols)) {
                    *(uint32_t*)rcode_at(i) = packed;
                    *rscale_at(i) = (uint8_t)rbyte;
                }
                __builtin_amdgcn_sched_barrier(0);
            }
        }

        // block maxima (as fp32 bit patterns): this thread's RPT rows, then
        // across the block's row groups
        uint32_t amax[CPT];
        if (IN_BF16) {
            // two columns per word: packed 16-bit maxima of the magnitudes
            u16x2_t cm[4];
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                cm[w] = __builtin_bit_cast(u16x2_t, v[0][w] & 0x7FFF7FFFu);
#pragma unroll
                for (int i = 1; i < RPT; ++i)
                    cm[w] = __builtin_elementwise_max(
                        cm[w], __builtin_bit_cast(u16x2_t, v[i][w] & 0x7FFF7FFFu));
            }
            if (NPB > 1) {
                *(uint4*)&part[NPB > 1 ? rg : 0][cg * 4] =
                    make_uint4(__builtin_bit_cast(uint32_t, cm[0]), __builtin_bit_cast(uint32_t, cm[1]),
                               __builtin_bit_cast(uint32_t, cm[2]), __builtin_bit_cast(uint32_t, cm[3]));
                __syncthreads();
                const int g0 = (rg / NPB) * NPB;
#pragma unroll
                for (int q = 0; q < NPB; ++q) {
                    const uint4 o = *(const uint4*)&part[NPB > 1 ? g0 + q : 0][cg * 4];
                    cm[0] = __builtin_elementwise_max(cm[0], __builtin_bit_cast(u16x2_t, o.x));
                    cm[1] = __builtin_elementwise_max(cm[1], __builtin_bit_cast(u16x2_t, o.y));
                    cm[2] = __builtin_elementwise_max(cm[2], __builtin_bit_cast(u16x2_t, o.z));
                    cm[3] = __builtin_elementwise_max(cm[3], __builtin_bit_cast(u16x2_t, o.w));
                }
            }
#pragma unroll
            for (int j = 0; j < CPT; ++j)
                amax[j] = (uint32_t)((j & 1) ? cm[j >> 1].y : cm[j >> 1].x) << 16;
        } else {
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                uint32_t m = 0;
#pragma unroll
                for (int i = 0; i < RPT; ++i) m = max(m, col_bits(i, j) & 0x7FFFFFFFu);
                amax[j] = m;
            }
            if (NPB > 1) {
#pragma unroll
                for (int j = 0; j < CPT; ++j) part[NPB > 1 ? rg : 0][cg * CPT + j] = amax[j];
                __syncthreads();
                const int g0 = (rg / NPB) * NPB;
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    uint32_t m = 0;
#pragma unroll
                    for (int q = 0; q < NPB; ++q)
                        m = max(m, part[NPB > 1 ? g0 + q : 0][cg * CPT + j]);
                    amax[j] = m;
                }
            }
        }

        // RPT rows of each column -> RPT/2 code bytes (rows 2p, 2p+1 -> byte p)
        uint32_t out[CPT][WPT];
#pragma unroll
        for (int j = 0; j < CPT; ++j) {
            const BlockScale bs = block_scale(amax[j] >> 23);
            const uint32_t byte = bs.byte;
            const float sc = bs.sc;
#pragma unroll
            for (int q = 0; q < WPT; ++q) out[j][q] = 0;
            if (!SR) {
#pragma unroll
                for (int p = 0; p < RPT / 2; ++p) {
                    uint32_t& dst = out[j][p / 4];
                    if (IN_BF16) {
                        // column j of rows 2p (low half) and 2p+1 (high half): the
                        // low or high 16-bit halves of the two rows' words
                        const bf16x2_t pr = __builtin_bit_cast(
                            bf16x2_t, __builtin_amdgcn_perm(v[2 * p + 1][j >> 1], v[2 * p][j >> 1],
                                                            (j & 1) ? 0x07060302u : 0x05040100u));
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
#pragma unroll
            for (int q = 0; q < WPT; ++q) out[j][q] &= bs.keep;  // SR codes are filled in below
            if ((rg % NPB) == 0 && rows_ok) sst[cg * CPT + j][rg / NPB] = (uint8_t)byte;
        }
        if (SR) {
            // column j's 16-bit lane of row r is half j & 1 of word j / 2 of the
            // random words of positions r*cols + c0 .. +7
            float sc[CPT];
            uint32_t keep[CPT];
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                const BlockScale bs = block_scale(amax[j] >> 23);
                keep[j] = bs.keep;
                sc[j] = bs.sc;
            }
#pragma unroll
            for (int p = 0; p < RPT / 2; ++p) {
                const int64_t r = r0 + rg * RPT + 2 * p;
                uint32_t w0[4], w1[4];
                uint64_t q0 = (uint64_t)r * (uint64_t)cols + (uint64_t)c0 + rng_off;
                // keeps each pair's Philox chains in place (hoisting all of them
                // to the top of the loop multiplies the live registers)
                asm volatile("" : "+v"(q0));
                if (ALIGNED) {
                    // bf16: lanes 0..7 of counter q0 / 8; fp32: lanes 0..3 or 4..7
                    const uint64_t n0 = q0 >> 3, n1 = (q0 + (uint64_t)cols) >> 3;
                    const Philox4 a =
                        philox4x32_10((uint32_t)n0, (uint32_t)(n0 >> 32), 0u, 0u, k0, k1);
                    const Philox4 b =
                        philox4x32_10((uint32_t)n1, (uint32_t)(n1 >> 32), 0u, 0u, k0, k1);
                    const bool hi4 = !IN_BF16 && (q0 & 4);
#pragma unroll
                    for (int k = 0; k < 4; ++k) {
                        w0[k] = (IN_BF16 || k >= 2) ? a.v[k] : (hi4 ? a.v[k + 2] : a.v[k]);
                        w1[k] = (IN_BF16 || k >= 2) ? b.v[k] : (hi4 ? b.v[k + 2] : b.v[k]);
                    }
                } else {
                    sr_words8(q0, k0, k1, w0);
                    sr_words8(q0 + (uint64_t)cols, k0, k1, w1);
                }
#pragma unroll
                for (int j = 0; j < CPT; ++j) {
                    const uint32_t u0 = (w0[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
                    const uint32_t u1 = (w1[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
                    const uint32_t bt = sr_pair(as_f32(col_bits(2 * p, j)),
                                                as_f32(col_bits(2 * p + 1, j)), sc[j], u0 << 16,
                                                u1 << 15);
                    out[j][p / 4] |= (bt & keep[j]) << (8 * (p & 3));
                }
                if (ROW == 3) {
                    // the same words give rows 2p and 2p+1 their ROW codes
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        const int i = 2 * p + h;
                        const BlockScale bs = row_scale(i);
                        const uint32_t rbyte = bs.byte;
                        float xf[8];
#pragma unroll
                        for (int j = 0; j < 8; ++j)
                            xf[j] = (j & 1) ? bf16_hi(v[i][j >> 1]) : bf16_lo(v[i][j >> 1]);
                        const uint32_t packed = sr_pack8(xf, bs.sc, h ? w1 : w0) & bs.keep;
                        if (interior || (rows_ok && c0 < cols)) {
                            *(uint32_t*)rcode_at(i) = packed;
                            *rscale_at(i) = (uint8_t)rbyte;
                        }
                    }
                }
                // one row pair at a time: interleaving the pairs' Philox chains
                // only raises register pressure (and lowers occupancy)
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // stage: column cg*CPT + j, bytes rg*RPT/2 .. of its tile segment.
        // Every column's staged bytes start on the same LDS bank (the pitch
        // times CPT columns is a multiple of 128 bytes), so the 16-byte
        // chunks of column c sit rotated by (c / CPT) chunks: the lanes of
        // one write (16 column groups) then spread over the banks instead of
        // all hitting one; the reads below undo the rotation.
        constexpr int NCH = TR / 32;  // 16-byte chunks per staged column
        auto staged = [&](int col, int byte) -> uint8_t* {
            const int ch = ((byte >> 4) + col / CPT) & (NCH - 1);
            return cst + col * PITCH + ch * 16 + (byte & 15);
        };
        {
            // this thread's columns all have the rotation cg
            const int byte = rg * (RPT / 2);
            uint8_t* const w0 =
                cst + cg * CPT * PITCH + (((byte >> 4) + cg) & (NCH - 1)) * 16 + (byte & 15);
#pragma unroll
            for (int j = 0; j < CPT; ++j) {
                if (WPT == 2)
                    *(uint2*)(w0 + j * PITCH) = make_uint2(out[j][0], out[j][WPT - 1]);
                else
                    *(uint32_t*)(w0 + j * PITCH) = out[j][0];
            }
        }
        __syncthreads();

        // codes: each column's vrows/2 bytes, written by TR/32 consecutive lanes
        // with 16-byte stores when the column stride allows them
        const int64_t half_rows = rows / 2;
        const int vbytes = vrows / 2;
        const int64_t cbase = tcol * TC;
        constexpr int CH16 = TR / 32;  // 16-byte chunks per column segment
        // (k-th store of a thread: kThreads / CH16 columns further on, a
        // uniform step from the thread's first destination)
        uint8_t* const ccb = codes + cbase * half_rows + r0 / 2;  // uniform
        auto ccode_at = [&](int col, int byte) -> uint8_t* {
            const int64_t o = col * half_rows + byte;
            return ALIGNED ? ccb + (uint32_t)o : ccb + o;
        };
        if ((half_rows & 15) == 0) {
            const int col0 = tid / CH16, ch = tid % CH16;
#pragma unroll
            for (int k = 0; k < TC * CH16 / kThreads; ++k) {
                const int col = col0 + k * (kThreads / CH16);
                if (interior || (cbase + col < cols && ch * 16 < vbytes))
                    *(uint4*)ccode_at(col, ch * 16) = *(const uint4*)staged(col, ch * 16);
            }
        } else {
            const int col0 = tid / (2 * CH16), ch = tid % (2 * CH16);
#pragma unroll
            for (int k = 0; k < TC * 2 * CH16 / kThreads; ++k) {
                const int col = col0 + k * (kThreads / (2 * CH16));
                if (interior || (cbase + col < cols && ch * 8 < vbytes))
                    *(uint2*)ccode_at(col, ch * 8) = *(const uint2*)staged(col, ch * 8);
            }
        }
        // scales: each column's vrows/BLOCK bytes
        if (tid < TC) {
            const int64_t c = cbase + tid;
            if (c < cols) {
                const int nb = vrows / BLOCK;
                uint8_t* dst = scales + c * nrb + r0 / BLOCK;
                if (nb == BPT && BPT >= 4 && ((uintptr_t)dst % BPT) == 0) {
                    uint32_t w[BPT >= 4 ? BPT / 4 : 1];
#pragma unroll
                    for (int q = 0; q < BPT / 4; ++q)
                        w[q] = sst[tid][4 * q] | (sst[tid][4 * q + 1] << 8) |
                               (sst[tid][4 * q + 2] << 16) | ((uint32_t)sst[tid][4 * q + 3] << 24);
                    if (BPT == 8)
                        *(uint2*)dst = make_uint2(w[0], w[BPT / 4 - 1]);
                    else
#pragma unroll
                        for (int q = 0; q < BPT / 4; ++q) ((uint32_t*)dst)[q] = w[q];
                } else {
#pragma unroll
                    for (int b2 = 0; b2 < BPT; ++b2)
                        if (b2 < nb) dst[b2] = sst[tid][b2];
                }
            }
        }
    };

    uint32_t v[RPT][4];
    load(tile, v);
    process(tile, v);
}

// Rows per thread of the column-pass tile: 8 (a 128-row tile) for the fused
// passes and the stochastic ones, 16 (a 256-row tile, whole 128-byte lines
// of codes per column) for the nearest-even column pass alone.  The
// stochastic passes need the registers; the fused nearest-even ones measured
// 10-20% faster with 8 at the layer's X and W sizes (twice the workgroups
// overlap their load, convert and store phases); the column pass alone on
// the 13B-shaped weight (5120 x 13824) measured 35.6 us with 8 and 34.2 us
// with 16.
template <int SR, int ROW>
struct ColRows {
    static constexpr int value = (SR == 0 && ROW == 0) ? 16 : 8;
};

template <int IN_BF16, int SR, int AL, int ROW>
static hipError_t col_dispatch(int block, int64_t nct, hipStream_t s, const void* x, int64_t rows,
                               int64_t cols, int64_t ld, uint8_t* codes, uint8_t* scales,
                               uint32_t k0, uint32_t k1, uint64_t off, int64_t nrb,
                               uint8_t* codes_r = nullptr, uint8_t* scales_r = nullptr,
                               uint32_t kr0 = 0, uint32_t kr1 = 0,
                               const uint32_t* zmask = nullptr) {
    constexpr int RPT = ColRows<SR, ROW>::value;
    if (AL) {
        // the ALIGNED kernels address within a tile with 32-bit offsets
        constexpr int64_t kLim = (int64_t)1 << 31;
        const int64_t tc = IN_BF16 ? 128 : 64, es = IN_BF16 ? 2 : 4;
        if (16 * RPT * ld * es >= kLim || tc * (rows / 2) >= kLim || 16 * RPT * (cols / 2) >= kLim)
            return col_dispatch<IN_BF16, SR, 0, ROW>(block, nct, s, x, rows, cols, ld, codes, scales,
                                                     k0, k1, off, nrb, codes_r, scales_r, kr0, kr1,
                                                     zmask);
    }
    const int64_t nrt = (rows + 16 * RPT - 1) / (16 * RPT);
    const int64_t n_tiles = nrt * nct;
    if (n_tiles >= ((int64_t)1 << 31)) return hipErrorInvalidValue;
    const dim3 grid((unsigned)n_tiles);
    const FastDiv ctd = make_fastdiv((uint32_t)nct);
#define FP4Q_COL_LAUNCH(B)                                                                    \
    FP4Q_LAUNCH((quantize_col_kernel<IN_BF16, B, SR, AL, ROW, RPT>), grid, kThreads, 0, s,               \
        x, rows, cols, ld, codes, scales, k0, k1, off, nrb, ctd,                              \
        codes_r, scales_r, kr0, kr1, zmask)
    switch (block) {
        case 16: FP4Q_COL_LAUNCH(16); break;
        case 32: FP4Q_COL_LAUNCH(32); break;
        case 64: FP4Q_COL_LAUNCH(64); break;
        default: FP4Q_COL_LAUNCH(128); break;
    }
#undef FP4Q_COL_LAUNCH
    return hipGetLastError();
}

hipError_t launch_quantize_col(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld,
                               int block, bool sr, uint64_t seed, uint64_t off, uint8_t* codes,
                               uint8_t* scales, hipStream_t s, const uint32_t* zmask) {
    const int64_t cols_per_tile = dtype == BF16 ? 128 : 64;
    const int64_t nct = (cols + cols_per_tile - 1) / cols_per_tile;
    const int64_t nrb = rows / block;
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const bool al = (cols % 8) == 0 && (off % 8) == 0;
    if (dtype == BF16) {
        if (!sr)
            return (cols % 8) == 0
                       ? col_dispatch<1, 0, 1, 0>(block, nct, s, x, rows, cols, ld, codes, scales,
                                                  k0, k1, off, nrb, nullptr, nullptr, 0, 0, zmask)
                       : col_dispatch<1, 0, 0, 0>(block, nct, s, x, rows, cols, ld, codes, scales,
                                                  k0, k1, off, nrb, nullptr, nullptr, 0, 0, zmask);
        return al ? col_dispatch<1, 1, 1, 0>(block, nct, s, x, rows, cols, ld, codes, scales, k0,
                                             k1, off, nrb, nullptr, nullptr, 0, 0, zmask)
                  : col_dispatch<1, 1, 0, 0>(block, nct, s, x, rows, cols, ld, codes, scales, k0,
                                             k1, off, nrb, nullptr, nullptr, 0, 0, zmask);
    }
    if (!sr)
        return (cols % 8) == 0
                   ? col_dispatch<0, 0, 1, 0>(block, nct, s, x, rows, cols, ld, codes, scales, k0,
                                              k1, off, nrb, nullptr, nullptr, 0, 0, zmask)
                   : col_dispatch<0, 0, 0, 0>(block, nct, s, x, rows, cols, ld, codes, scales, k0,
                                              k1, off, nrb, nullptr, nullptr, 0, 0, zmask);
    return al ? col_dispatch<0, 1, 1, 0>(block, nct, s, x, rows, cols, ld, codes, scales, k0, k1,
                                         off, nrb, nullptr, nullptr, 0, 0, zmask)
              : col_dispatch<0, 1, 0, 0>(block, nct, s, x, rows, cols, ld, codes, scales, k0, k1,
                                         off, nrb, nullptr, nullptr, 0, 0, zmask);
}

// Both quantisations of a bf16 tensor in one pass (rows and cols multiples
// of the block): ROW blocks into codes_r/scales_r, COL blocks into
// codes_c/scales_c, each exactly as its own launch would write them.
hipError_t launch_quantize_dual(const void* x, int64_t rows, int64_t cols, int64_t ld, int block,
                                bool sr_row, uint64_t seed_row, bool sr_col, uint64_t seed_col,
                                uint64_t off, uint8_t* codes_r, uint8_t* scales_r,
                                uint8_t* codes_c, uint8_t* scales_c, hipStream_t s) {
    const int64_t nct = (cols + 127) / 128;
    const int64_t nrb = rows / block;
    const uint32_t k0 = (uint32_t)seed_col, k1 = (uint32_t)(seed_col >> 32);
    const uint32_t kr0 = (uint32_t)seed_row, kr1 = (uint32_t)(seed_row >> 32);
    const bool al = (cols % 8) == 0 && (off % 8) == 0;
#define FP4Q_DUAL(SRC, AL, ROW)                                                                 \
    return col_dispatch<1, SRC, AL, ROW>(block, nct, s, x, rows, cols, ld, codes_c, scales_c, k0, \
                                         k1, off, nrb, codes_r, scales_r, kr0, kr1)
    const bool shared = sr_row && sr_col && seed_row == seed_col;
    if (al) {
        if (sr_col) {
            if (shared) FP4Q_DUAL(1, 1, 3);
            if (sr_row) FP4Q_DUAL(1, 1, 2);
            FP4Q_DUAL(1, 1, 1);
        }
        if (sr_row) FP4Q_DUAL(0, 1, 2);
        FP4Q_DUAL(0, 1, 1);
    }
    if (sr_col) {
        if (shared) FP4Q_DUAL(1, 0, 3);
        if (sr_row) FP4Q_DUAL(1, 0, 2);
        FP4Q_DUAL(1, 0, 1);
    }
    if (sr_row) FP4Q_DUAL(0, 0, 2);
    FP4Q_DUAL(0, 0, 1);
#undef FP4Q_DUAL
}

// ---------------------------------------------------------------------------
// Channel masks for the quantisers' zero mask: a fill, then one atomic OR per
// listed index (two launches on the stream, so the OR follows the fill).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kThreads) void mask_fill_kernel(uint32_t* __restrict__ mask,
                                                             int64_t words) {
    const int64_t i = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (i < words) mask[i] = 0u;
}

__global__ __launch_bounds__(kThreads) void mask_set_kernel(const int32_t* __restrict__ idx,
                                                            int32_t n, int64_t length,
                                                            uint32_t* __restrict__ mask) {
    const int64_t t = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (t >= n) return;
    const int64_t c = idx[t];
    if (c < 0 || c >= length) return;  // outside the axis: ignored
    atomicOr(mask + (c >> 5), 1u << (c & 31));
}

hipError_t launch_channel_mask(const int32_t* idx, int32_t n, int64_t length, uint32_t* mask,
                               hipStream_t s) {
    const int64_t words = (length + 31) / 32;
    FP4Q_LAUNCH((mask_fill_kernel), dim3((unsigned)((words + kThreads - 1) / kThreads)), kThreads, 0, s,
        mask, words);
    if (n > 0)
        FP4Q_LAUNCH((mask_set_kernel), dim3((unsigned)((n + kThreads - 1) / kThreads)), kThreads, 0, s,
            idx, n, length, mask);
    return hipGetLastError();
}

}  // namespace fp4q
