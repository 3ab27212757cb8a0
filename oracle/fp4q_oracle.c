/*
 * fp4q_oracle.c -- plain, slow, single-threaded CPU oracle for the block-scaled
 * MXFP4 linear-layer hot path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product library links, calls or
 * includes this file; only the test-suite, the smoke check and the CPU-baseline
 * leg of the benchmark load it.  It shares no code, header, table or constant
 * generator with the HIP kernels.
 *
 * Every quantity is computed from its plain definition in double precision
 * (which is exact for every step below except the DGE power function and the
 * GEMM/HCP sums).  Sources, by page and section:
 *
 *   [P1] aicoding.csdn.net tutorial on quantisation gradients and MXFP4
 *        ("深度学习中的梯度计算基础 ... MXFP4格式的独特设计"):
 *        sec. 2.1 Q(x) = s*round(x/s); sec. 3.1 STE dQ/dx ~ 1;
 *        sec. 4.1 block-structured shared scale over 16..128 elements.
 *   [P2] framerc.cn overview of low-precision training ("低精度训练技术概述"):
 *        sec. 1.1 E8M0 = 8 exponent bits, 0 mantissa bits;
 *        sec. 3.2 stochastic rounding: round up with probability equal to
 *        the fractional distance (read here at 16-bit resolution as the
 *        carry rule of orc_sr_code, which is rand < frac with rand the
 *        complement of the 16 random bits and frac truncated to 16 bits).
 *   [P3] devpress.csdn.net "大模型4位训练中的异常值动态分析与优化实践":
 *        sec. 1.1 E2M1 covers [-6, 6]; sec. 3.1 HCP error decomposition and
 *        the dual-kernel (D) mode; sec. 3.2 hcp_gemm sketch; sec. 4.1 top 9%.
 *   [P4] lsdiaocha.cn summary of the MSRA FP4-training paper (arXiv 2501.17116):
 *        sec. 一 E2M1 (2 exponent bits, 1 mantissa bit, range -6..6);
 *        sec. 二 DGE f(x) = d/2 (1 + sign(2x/d - 1) |2x/d - 1|^(1/k)) and the
 *        clamp of its derivative at 3.0.
 *
 * Readings of points the pages leave open (E8M0 bias, exponent rule, tie rule,
 * saturation, sign of zero, SR in magnitude form, RNG, DGE beyond the grid,
 * HCP residual content) are fixed by readings of this implementation, and
 * the code below states each where it is used.
 *
 * Philox4x32 follows Salmon, Moraes, Dror, Shaw, "Parallel Random Numbers:
 * As Easy as 1, 2, 3" (SC'11), written from that paper's description.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#define ORC_F32 0
#define ORC_BF16 1
#define ORC_ROW 0
#define ORC_COL 1
#define ORC_RNE 0
#define ORC_SR 1
#define ORC_STE 0
#define ORC_DGE 1

/* Rounds of Philox4x32 used for stochastic rounding (the published default). */
#define ORC_PHILOX_ROUNDS 10

/* ------------------------------------------------------------------------- */
/* Element formats                                                           */
/* ------------------------------------------------------------------------- */

/* E2M1 magnitudes by 3-bit code: sign | e1 e0 | m with exponent bias 1 and a
 * subnormal at e = 0.  This is the only 1-2-1 layout whose largest magnitude
 * is 6, the range [P3 sec. 1.1] and [P4 sec. 一] give. */
static const double E2M1_MAG[8] = {0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0};

double orc_e2m1_value(int code) {
    double v = E2M1_MAG[code & 7];
    return (code & 8) ? -v : v;
}

static uint32_t f32_bits(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return u;
}
static float bits_f32(uint32_t u) {
    float f;
    memcpy(&f, &u, 4);
    return f;
}

/* Load element i of a bf16 or fp32 array as its fp32 bit pattern (bf16 -> fp32
 * is exact: the bf16 bits are the top half of the fp32 bits). */
static uint32_t load_bits(const void* p, int dtype, int64_t i) {
    if (dtype == ORC_BF16) return ((uint32_t)((const uint16_t*)p)[i]) << 16;
    return ((const uint32_t*)p)[i];
}

/* E8M0 byte for a block with largest magnitude amax (given as fp32 bits with
 * the sign cleared).  The scale is 2^e with e = floor(log2 amax) - 2, clamped
 * below at -127; byte = e + 127 (the bias equals fp32's, [P2 sec. 1.1] gives
 * only "8 exponent bits, no mantissa").  floor(log2) is read from the bits:
 * biased exponent - 127 for normals, -149 + index of the top set mantissa
 * bit for subnormals.  amax = 0 gives byte 0.  A non-finite amax gives 0xFF.
 * Returns the byte. */
int orc_e8m0_byte(uint32_t amax_bits) {
    uint32_t ex = (amax_bits >> 23) & 0xFF;
    uint32_t man = amax_bits & 0x7FFFFF;
    int fl;
    if (ex == 0xFF) return 0xFF;
    if (ex == 0 && man == 0) return 0;
    if (ex != 0) {
        fl = (int)ex - 127;
    } else {
        int h = 22;
        while (!(man & (1u << h))) --h;
        fl = h - 149;
    }
    int e = fl - 2;
    if (e < -127) e = -127;
    if (e > 127) e = 127;
    return e + 127;
}

/* Round-to-nearest onto the E2M1 grid with saturation; y = x / 2^e exactly.
 * Ties go to the even code (mantissa bit 0): 0.25->0, 0.75->1, 1.25->1,
 * 1.75->2, 2.5->2, 3.5->4, 5->4.  |y| > 6 saturates to 6.  The sign bit is
 * always kept, so a negative value that rounds to zero is code 0x8. */
int orc_rne_code(double y) {
    int sign = signbit(y) ? 8 : 0;
    double m = fabs(y);
    int best = 0;
    if (m >= 6.0) {
        best = 7;
    } else {
        double bd = INFINITY;
        for (int c = 0; c < 8; ++c) {
            double d = fabs(m - E2M1_MAG[c]);
            /* strictly closer wins; an exact tie picks the even code */
            if (d < bd || (d == bd && (c & 1) == 0)) {
                bd = d;
                best = c;
            }
        }
    }
    return sign | best;
}

/* Stochastic rounding on the E2M1 grid, magnitude form of "round up with
 * probability equal to the fractional distance" ([P2 sec. 3.2]) at 16-bit
 * resolution: lo = largest grid value <= |y|, hi = the next one,
 * frac = (|y| - lo) / (hi - lo); the fraction truncated to 16 bits and the
 * 16 random bits are added, and a carry out of 16 bits rounds up:
 * round up iff u16 + floor(frac * 2^16) >= 2^16, so P(up) =
 * floor(frac * 2^16) / 2^16, within 2^-16 of frac (every quantity is exact in
 * double).  Written as the page's comparison this is rand < frac with
 * rand = (0xFFFF - u16) / 2^16 and frac truncated to 16 bits; it is not
 * u16 < frac * 2^16, which rounds a given u16 differently on up to ~90% of
 * the 2^16 values (the two draws are complements of each other).
 * |y| >= 6 gives 6. */
int orc_sr_code(double y, uint32_t u16) {
    int sign = signbit(y) ? 8 : 0;
    double m = fabs(y);
    if (m >= 6.0) return sign | 7;
    int lo = 0;
    while (lo < 7 && E2M1_MAG[lo + 1] <= m) ++lo;
    double frac = (m - E2M1_MAG[lo]) / (E2M1_MAG[lo + 1] - E2M1_MAG[lo]);
    int up = ((double)u16 + floor(frac * 65536.0) >= 65536.0);
    return sign | (lo + up);
}

/* ------------------------------------------------------------------------- */
/* Philox4x32 (Salmon et al., SC'11)                                          */
/* ------------------------------------------------------------------------- */

/* One call: counter (4 words) and key (2 words) through `rounds` rounds.  Each
 * round multiplies words 0 and 2 by the two Philox multipliers, takes the high
 * and low halves of the 64-bit products, and mixes them with words 1 and 3
 * and the round key; the key is bumped by the two Weyl constants between
 * rounds. */
void orc_philox4x32(const uint32_t ctr_in[4], const uint32_t key_in[2], int rounds,
                    uint32_t out[4]) {
    const uint32_t M0 = 0xD2511F53u, M1 = 0xCD9E8D57u;
    const uint32_t W0 = 0x9E3779B9u, W1 = 0xBB67AE85u;
    uint32_t c0 = ctr_in[0], c1 = ctr_in[1], c2 = ctr_in[2], c3 = ctr_in[3];
    uint32_t k0 = key_in[0], k1 = key_in[1];
    for (int r = 0; r < rounds; ++r) {
        if (r > 0) {
            k0 += W0;
            k1 += W1;
        }
        uint64_t p0 = (uint64_t)M0 * c0;
        uint64_t p1 = (uint64_t)M1 * c2;
        uint32_t hi0 = (uint32_t)(p0 >> 32), lo0 = (uint32_t)p0;
        uint32_t hi1 = (uint32_t)(p1 >> 32), lo1 = (uint32_t)p1;
        uint32_t n0 = hi1 ^ c1 ^ k0;
        uint32_t n1 = lo1;
        uint32_t n2 = hi0 ^ c3 ^ k1;
        uint32_t n3 = lo0;
        c0 = n0;
        c1 = n1;
        c2 = n2;
        c3 = n3;
    }
    out[0] = c0;
    out[1] = c1;
    out[2] = c2;
    out[3] = c3;
}

/* 16 random bits for logical position pos = element index + rng offset.
 * One Philox call serves 8 consecutive positions: counter = (pos >> 3) as a
 * 64-bit value in words 0..1, words 2..3 zero; key = the 64-bit seed.  Position
 * pos takes 16-bit half (pos & 1) of output word (pos & 7) >> 1. */
uint32_t orc_sr_bits(uint64_t seed, uint64_t pos) {
    uint64_t n = pos >> 3;
    uint32_t ctr[4] = {(uint32_t)n, (uint32_t)(n >> 32), 0u, 0u};
    uint32_t key[2] = {(uint32_t)seed, (uint32_t)(seed >> 32)};
    uint32_t out[4];
    orc_philox4x32(ctr, key, ORC_PHILOX_ROUNDS, out);
    int lane = (int)(pos & 7);
    return (out[lane >> 1] >> (16 * (lane & 1))) & 0xFFFFu;
}

/* ------------------------------------------------------------------------- */
/* Quantize / dequantize                                                      */
/* ------------------------------------------------------------------------- */

/* Source element (r, c) of a [rows, cols] tensor with row stride ld. */
static uint32_t src_bits(const void* x, int dtype, int64_t ld, int64_t r, int64_t c) {
    return load_bits(x, dtype, r * ld + c);
}

/* Quantize one block of b elements whose fp32 bit patterns are in v[] and
 * whose logical source indices are idx[].  Writes b codes (unpacked) and
 * returns the scale byte. */
static int quantize_block(const uint32_t* v, const uint64_t* idx, int b, int round,
                          uint64_t seed, uint64_t off, uint8_t* code_out) {
    uint32_t amax = 0;
    int nonfinite = 0;
    for (int t = 0; t < b; ++t) {
        uint32_t a = v[t] & 0x7FFFFFFFu;
        if ((a >> 23) == 0xFF) nonfinite = 1;
        if (a > amax) amax = a; /* |x| ordering equals bit ordering */
    }
    if (nonfinite) {
        for (int t = 0; t < b; ++t) code_out[t] = 0;
        return 0xFF;
    }
    int byte = orc_e8m0_byte(amax);
    int e = byte - 127;
    for (int t = 0; t < b; ++t) {
        double x = (double)bits_f32(v[t]);
        double y = ldexp(x, -e); /* exact in double */
        if (round == ORC_RNE)
            code_out[t] = (uint8_t)orc_rne_code(y);
        else
            code_out[t] = (uint8_t)orc_sr_code(y, orc_sr_bits(seed, idx[t] + off));
    }
    return byte;
}

/* Quantize a [rows, cols] tensor (row stride ld, bf16 or fp32).
 *   axis ROW: block j of row r = columns [j*b, (j+1)*b);
 *             codes [rows, cols/2], scales [rows, cols/b].
 *   axis COL: block j of column c = rows [j*b, (j+1)*b);
 *             codes [cols, rows/2] (K-major), scales [cols, rows/b].
 * Two codes per byte, the lower index along the block axis in the low nibble.
 * Returns 0, or -1 on a shape the oracle does not take. */
int orc_quantize(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int block,
                 int axis, int round, uint64_t seed, uint64_t rng_offset, uint8_t* codes,
                 uint8_t* scales) {
    if (block <= 0 || block % 2) return -1;
    if (axis == ORC_ROW && cols % block) return -1;
    if (axis == ORC_COL && rows % block) return -1;
    uint32_t* v = (uint32_t*)malloc(sizeof(uint32_t) * block);
    uint64_t* idx = (uint64_t*)malloc(sizeof(uint64_t) * block);
    uint8_t* cd = (uint8_t*)malloc(block);
    if (axis == ORC_ROW) {
        int64_t nb = cols / block;
        for (int64_t r = 0; r < rows; ++r)
            for (int64_t j = 0; j < nb; ++j) {
                for (int t = 0; t < block; ++t) {
                    int64_t c = j * block + t;
                    v[t] = src_bits(x, dtype, ld, r, c);
                    idx[t] = (uint64_t)(r * cols + c);
                }
                scales[r * nb + j] = (uint8_t)quantize_block(v, idx, block, round, seed,
                                                             rng_offset, cd);
                for (int t = 0; t < block; t += 2)
                    codes[r * (cols / 2) + (j * block + t) / 2] =
                        (uint8_t)((cd[t] & 0xF) | ((cd[t + 1] & 0xF) << 4));
            }
    } else {
        int64_t nb = rows / block;
        for (int64_t c = 0; c < cols; ++c)
            for (int64_t j = 0; j < nb; ++j) {
                for (int t = 0; t < block; ++t) {
                    int64_t r = j * block + t;
                    v[t] = src_bits(x, dtype, ld, r, c);
                    idx[t] = (uint64_t)(r * cols + c);
                }
                scales[c * nb + j] = (uint8_t)quantize_block(v, idx, block, round, seed,
                                                             rng_offset, cd);
                for (int t = 0; t < block; t += 2)
                    codes[c * (rows / 2) + (j * block + t) / 2] =
                        (uint8_t)((cd[t] & 0xF) | ((cd[t + 1] & 0xF) << 4));
            }
    }
    free(v);
    free(idx);
    free(cd);
    return 0;
}

/* Two-dimensional block scaling ([P3] sec. 4.1: the backward pass of the
 * recipe uses 2D block scales): every tile x tile square of X is one block
 * (one shared scale from the square's amax, its tile*tile elements coded as
 * any block), and the same codes are written in both layouts, so the ROW
 * (blocks along columns) and the COL (blocks along rows, K-major) forms hold
 * the same values and W and its transpose share one quantisation.
 *   codes_r [rows, cols/2], scales_r [rows, cols/tile] (the square's scale
 *   repeated on each of its rows); codes_c [cols, rows/2], scales_c
 *   [cols, rows/tile].  SR draws element (r, c) from counter r*cols + c as
 *   orc_quantize does.  Returns 0, or -1 on a shape the oracle does not take. */
int orc_quantize_2d(const void* x, int dtype, int64_t rows, int64_t cols, int64_t ld, int tile,
                    int round, uint64_t seed, uint64_t rng_offset, uint8_t* codes_r,
                    uint8_t* scales_r, uint8_t* codes_c, uint8_t* scales_c) {
    if (tile <= 0 || tile % 2 || rows % tile || cols % tile) return -1;
    const int b = tile * tile;
    uint32_t* v = (uint32_t*)malloc(sizeof(uint32_t) * b);
    uint64_t* idx = (uint64_t*)malloc(sizeof(uint64_t) * b);
    uint8_t* cd = (uint8_t*)malloc(b);
    for (int64_t tr = 0; tr < rows / tile; ++tr)
        for (int64_t tc = 0; tc < cols / tile; ++tc) {
            for (int i = 0; i < tile; ++i)
                for (int j = 0; j < tile; ++j) {
                    int64_t r = tr * tile + i, c = tc * tile + j;
                    v[i * tile + j] = src_bits(x, dtype, ld, r, c);
                    idx[i * tile + j] = (uint64_t)(r * cols + c);
                }
            uint8_t byte = (uint8_t)quantize_block(v, idx, b, round, seed, rng_offset, cd);
            for (int i = 0; i < tile; ++i) {
                int64_t r = tr * tile + i;
                scales_r[r * (cols / tile) + tc] = byte;
                for (int j = 0; j < tile; j += 2)
                    codes_r[r * (cols / 2) + (tc * tile + j) / 2] =
                        (uint8_t)((cd[i * tile + j] & 0xF) | ((cd[i * tile + j + 1] & 0xF) << 4));
            }
            for (int j = 0; j < tile; ++j) {
                int64_t c = tc * tile + j;
                scales_c[c * (rows / tile) + tr] = byte;
                for (int i = 0; i < tile; i += 2)
                    codes_c[c * (rows / 2) + (tr * tile + i) / 2] =
                        (uint8_t)((cd[i * tile + j] & 0xF) | ((cd[(i + 1) * tile + j] & 0xF) << 4));
            }
        }
    free(v);
    free(idx);
    free(cd);
    return 0;
}

/* Value of packed element (r, k) of a quantized [rows, kdim] operand. */
static double deq_elem(const uint8_t* codes, const uint8_t* scales, int64_t kdim, int block,
                       int64_t r, int64_t k) {
    uint8_t byte = codes[r * (kdim / 2) + k / 2];
    int code = (k & 1) ? (byte >> 4) : (byte & 0xF);
    int sb = scales[r * (kdim / block) + k / block];
    if (sb == 0xFF) return NAN;
    return ldexp(orc_e2m1_value(code), sb - 127);
}

/* Dequantize codes [rows, k/2] + scales [rows, k/block] to doubles [rows, k]:
 * value(code) * 2^(byte - 127), exact; byte 0xFF gives NaN. */
void orc_dequantize(const uint8_t* codes, const uint8_t* scales, int64_t rows, int64_t k,
                    int block, double* out) {
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < k; ++c) out[r * k + c] = deq_elem(codes, scales, k, block, r, c);
}

/* ------------------------------------------------------------------------- */
/* Rounding of double results to the output dtypes                            */
/* ------------------------------------------------------------------------- */

/* IEEE round-to-nearest-even of a double to fp32 (C conversion). */
void orc_round_f32(const double* in, float* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = (float)in[i];
}

/* Round-to-nearest-even of a double straight to bf16 (no detour through fp32,
 * which could round twice).  bf16 keeps 8 significant bits; its subnormal
 * quantum is 2^-133; magnitudes that round past the largest finite value
 * become infinity. */
uint16_t orc_bf16_from_double(double v) {
    if (isnan(v)) return 0x7FC0;
    uint16_t sign = signbit(v) ? 0x8000 : 0;
    double a = fabs(v);
    if (a == 0.0) return sign;
    if (isinf(a)) return sign | 0x7F80;
    int ex;
    frexp(a, &ex); /* a = f * 2^ex, f in [0.5, 1) */
    int q = ex - 8;
    if (q < -133) q = -133;
    double r = ldexp(rint(ldexp(a, -q)), q); /* rint: ties to even */
    if (r >= 0x1p128) return sign | 0x7F80;
    uint32_t b = f32_bits((float)r); /* r is exact in bf16, hence in fp32 */
    return (uint16_t)(sign | (b >> 16));
}

void orc_round_bf16(const double* in, uint16_t* out, int64_t n) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_bf16_from_double(in[i]);
}

/* ------------------------------------------------------------------------- */
/* Gradient estimators                                                        */
/* ------------------------------------------------------------------------- */

/* Width and lower end of the E2M1 interval holding m in [0, 6]: width 0.5 on
 * [0, 2), 1 on [2, 4), 2 on [4, 6]; m = 6 belongs to [4, 6]. */
static void e2m1_interval(double m, double* lo, double* delta) {
    if (m < 2.0) {
        *delta = 0.5;
    } else if (m < 4.0) {
        *delta = 1.0;
    } else {
        *delta = 2.0;
    }
    double l = floor(m / *delta) * *delta;
    if (m >= 6.0) l = 4.0;
    *lo = l;
}

/* DGE smooth staircase on one interval [P4 sec. 二]: t = offset from the
 * interval's lower end, delta = its width, k = sharpness.
 * f(t) = delta/2 * (1 + sign(2t/delta - 1) * |2t/delta - 1|^(1/k)). */
double orc_dge_f(double t, double delta, double k) {
    double u = 2.0 * t / delta - 1.0;
    double s = (u > 0) - (u < 0);
    return delta / 2.0 * (1.0 + s * pow(fabs(u), 1.0 / k));
}

/* Its derivative df/dt = (1/k) |u|^(1/k - 1) with u = 2t/delta - 1, clamped
 * above at clamp_max [P4 sec. 二].  At u = 0 the unclamped derivative is
 * infinite for k > 1 (so the clamp applies) and 1 for k = 1. */
double orc_dge_fprime(double t, double delta, double k, double clamp_max) {
    double u = 2.0 * t / delta - 1.0;
    double d = (1.0 / k) * pow(fabs(u), 1.0 / k - 1.0); /* pow(0, <0) = +inf */
    return d < clamp_max ? d : clamp_max;
}

/* Derivative factor for one element x whose block exponent is e (byte - 127):
 * m = |x| / 2^e; m > 6 (saturated) gives 1, the STE fallback; otherwise the
 * clamped DGE derivative on the interval holding m.  A non-finite block gives
 * NaN. */
static double dge_factor(double x, int byte, double k, double clamp_max) {
    if (byte == 0xFF) return NAN;
    double m = fabs(ldexp(x, -(byte - 127)));
    if (m > 6.0) return 1.0;
    double lo, delta;
    e2m1_interval(m, &lo, &delta);
    return orc_dge_fprime(m - lo, delta, k, clamp_max);
}

/* Gradient estimate for a [rows, cols] tensor.  STE: d = 1 [P1 sec. 3.1].
 * DGE: d from x's own block scales (same block axis as its quantization,
 * recomputed here).  Writes the factor d and the exact product g * d, both in
 * double, dense [rows, cols] (x and g are dense with row stride cols). */
int orc_grad_estimate(int mode, const void* x, int x_dtype, const void* g, int g_dtype,
                      int64_t rows, int64_t cols, int block, int axis, double k,
                      double clamp_max, double* d_out, double* out) {
    if (mode == ORC_STE) {
        for (int64_t i = 0; i < rows * cols; ++i) {
            d_out[i] = 1.0;
            out[i] = (double)bits_f32(load_bits(g, g_dtype, i));
        }
        return 0;
    }
    if (axis == ORC_ROW && cols % block) return -1;
    if (axis == ORC_COL && rows % block) return -1;
    for (int64_t r = 0; r < rows; ++r)
        for (int64_t c = 0; c < cols; ++c) {
            /* scale byte of the block holding (r, c) */
            uint32_t amax = 0;
            int nonfinite = 0;
            for (int t = 0; t < block; ++t) {
                int64_t rr = axis == ORC_ROW ? r : (r / block) * block + t;
                int64_t cc = axis == ORC_ROW ? (c / block) * block + t : c;
                uint32_t a = load_bits(x, x_dtype, rr * cols + cc) & 0x7FFFFFFFu;
                if ((a >> 23) == 0xFF) nonfinite = 1;
                if (a > amax) amax = a;
            }
            int byte = nonfinite ? 0xFF : orc_e8m0_byte(amax);
            double xv = (double)bits_f32(load_bits(x, x_dtype, r * cols + c));
            double gv = (double)bits_f32(load_bits(g, g_dtype, r * cols + c));
            double d = dge_factor(xv, byte, k, clamp_max);
            d_out[r * cols + c] = d;
            out[r * cols + c] = gv * d;
        }
    return 0;
}

/* ------------------------------------------------------------------------- */
/* FP4 x FP4 GEMM with per-block scales                                       */
/* ------------------------------------------------------------------------- */

/* C[i,j] = sum_k deq(a[i,k]) * deq(b[j,k]) in double, with S[i,j] =
 * sum_k |deq(a[i,k]) * deq(b[j,k])| for the error bound.  A: codes [M, K/2],
 * scales [M, K/32]; B: codes [N, K/2], scales [N, K/32] (both K-major). */
void orc_gemm(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
              const uint8_t* bc, const uint8_t* bs, int block, double* C, double* S) {
    double* arow = (double*)malloc(sizeof(double) * K);
    for (int64_t i = 0; i < M; ++i) {
        for (int64_t k = 0; k < K; ++k) arow[k] = deq_elem(ac, as, K, block, i, k);
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0, sab = 0.0;
            for (int64_t k = 0; k < K; ++k) {
                double p = arow[k] * deq_elem(bc, bs, K, block, j, k);
                acc += p;
                sab += fabs(p);
            }
            C[i * N + j] = acc;
            S[i * N + j] = sab;
        }
    }
    free(arow);
}

/* The same sum, entry by entry, for n sampled positions (ii[t], jj[t]). */
void orc_gemm_entries(int64_t K, const uint8_t* ac, const uint8_t* as, const uint8_t* bc,
                      const uint8_t* bs, int block, int64_t n, const int64_t* ii,
                      const int64_t* jj, double* C, double* S) {
    for (int64_t t = 0; t < n; ++t) {
        double acc = 0.0, sab = 0.0;
        for (int64_t k = 0; k < K; ++k) {
            double p = deq_elem(ac, as, K, block, ii[t], k) * deq_elem(bc, bs, K, block, jj[t], k);
            acc += p;
            sab += fabs(p);
        }
        C[t] = acc;
        S[t] = sab;
    }
}

/* Second formulation: each block's dot product summed exactly in integers on
 * doubled magnitudes (2|v| in {0,1,2,3,4,6,8,12}), then scaled by
 * 2^(ea + eb - 256) and added in double.  A 0xFF scale gives NaN. */
void orc_gemm_intblock(int64_t M, int64_t N, int64_t K, const uint8_t* ac, const uint8_t* as,
                       const uint8_t* bc, const uint8_t* bs, int block, double* C) {
    static const int TWICE[8] = {0, 1, 2, 3, 4, 6, 8, 12};
    int64_t nb = K / block;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double acc = 0.0;
            for (int64_t bb = 0; bb < nb; ++bb) {
                int ea = as[i * nb + bb], eb = bs[j * nb + bb];
                long isum = 0;
                for (int64_t k = bb * block; k < (bb + 1) * block; ++k) {
                    uint8_t ba = ac[i * (K / 2) + k / 2], bbyte = bc[j * (K / 2) + k / 2];
                    int ca = (k & 1) ? ba >> 4 : ba & 0xF;
                    int cb = (k & 1) ? bbyte >> 4 : bbyte & 0xF;
                    int va = TWICE[ca & 7] * ((ca & 8) ? -1 : 1);
                    int vb = TWICE[cb & 7] * ((cb & 8) ? -1 : 1);
                    isum += (long)va * vb;
                }
                if (ea == 0xFF || eb == 0xFF)
                    acc += NAN;
                else
                    acc += ldexp((double)isum, ea + eb - 256);
            }
            C[i * N + j] = acc;
        }
}

/* ------------------------------------------------------------------------- */
/* Hot-channel residual (dual-kernel mode)                                    */
/* ------------------------------------------------------------------------- */

/* Exact hot-channel correction of the quantized product, from the error
 * decomposition of [P3 sec. 3.1]: for output (i, j),
 *   R = sum_{c in H} ( X[i,c] W[c,j] - Xq[i,c] Wq[c,j] ),
 * which replaces, on the hot channels, the quantized operands' product by the
 * bf16 operands' product (all first- and second-order error terms of both
 * operands on H).  X: bf16 [M, K] (row stride K).  Xq: codes [M, K/2] +
 * scales [M, K/32].  W: bf16 [K, N] (row stride N).  Wq: K-major codes
 * [N, K/2] + scales [N, K/32].  Computed for n sampled (ii, jj) positions;
 * S gets sum |X W| + |Xq Wq| over H. */
void orc_hcp_residual_entries(int64_t N, int64_t K, const uint16_t* x, const uint8_t* xqc,
                              const uint8_t* xqs, const uint16_t* w, const uint8_t* wqc,
                              const uint8_t* wqs, const int32_t* hot, int32_t n_hot, int64_t n,
                              const int64_t* ii, const int64_t* jj, double* R, double* S) {
    for (int64_t t = 0; t < n; ++t) {
        int64_t i = ii[t], j = jj[t];
        double acc = 0.0, sab = 0.0;
        for (int32_t h = 0; h < n_hot; ++h) {
            int64_t c = hot[h];
            double xv = (double)bits_f32(((uint32_t)x[i * K + c]) << 16);
            double wv = (double)bits_f32(((uint32_t)w[c * N + j]) << 16);
            double xq = deq_elem(xqc, xqs, K, 32, i, c);
            double wq = deq_elem(wqc, wqs, K, 32, j, c);
            acc += xv * wv - xq * wq;
            sab += fabs(xv * wv) + fabs(xq * wq);
        }
        R[t] = acc;
        S[t] = sab;
    }
}

/* ------------------------------------------------------------------------- */
/* Bulk element helpers (loops over the scalar definitions above, so tests    */
/* can sweep millions of inputs through one call)                             */
/* ------------------------------------------------------------------------- */

void orc_e8m0_bytes(const uint32_t* amax_bits, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_e8m0_byte(amax_bits[i] & 0x7FFFFFFFu);
}

void orc_rne_codes(const double* y, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_rne_code(y[i]);
}

void orc_sr_codes(const double* y, const uint32_t* u16, int64_t n, uint8_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = (uint8_t)orc_sr_code(y[i], u16[i]);
}

void orc_sr_bits_range(uint64_t seed, uint64_t pos0, int64_t n, uint32_t* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_sr_bits(seed, pos0 + (uint64_t)i);
}

void orc_dge_f_many(const double* t, const double* delta, int64_t n, double k, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_dge_f(t[i], delta[i], k);
}

void orc_dge_fprime_many(const double* t, const double* delta, int64_t n, double k,
                         double clamp_max, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = orc_dge_fprime(t[i], delta[i], k, clamp_max);
}
