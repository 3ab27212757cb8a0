// Device-side helpers shared by the libfp4q kernels (gfx950 only).
//
// Element format: E2M1 (sign | 2 exponent bits | 1 mantissa bit, magnitudes
// 0, 0.5, 1, 1.5, 2, 3, 4, 6) with an E8M0 power-of-two block scale; two codes
// per byte, lower index in the low nibble (MSRA FP4-training summary page,
// sec. 一; outlier-dynamics page, sec. 1.1; low-precision overview page,
// sec. 1.1).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp4q {

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));

__device__ __forceinline__ float as_f32(uint32_t u) { return __uint_as_float(u); }
__device__ __forceinline__ uint32_t as_u32(float f) { return __float_as_uint(f); }

// fp32 value of the low / high bf16 of a packed pair (exact).
// 16-byte store with the non-temporal hint, for outputs this path does not
// read back soon (a dequantised or gradient tensor): they then do not
// displace data in the caches that the next kernels read.
__device__ __forceinline__ void store_nt(uint4* p, uint4 v) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    __builtin_nontemporal_store((v4u){v.x, v.y, v.z, v.w}, (v4u*)p);
}

// 16-byte load with the non-temporal hint, for inputs a kernel reads once:
// a streaming read of a tensor that is not in the caches runs faster with it
// (the ROW quantiser on an 8192 x 5632 bf16 tensor: 6.0 against 5.5 TB/s).
__device__ __forceinline__ uint4 load_nt(const void* p) {
    typedef unsigned int v4u __attribute__((ext_vector_type(4)));
    const v4u v = __builtin_nontemporal_load((const v4u*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

__device__ __forceinline__ float bf16_lo(uint32_t w) { return as_f32(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return as_f32(w & 0xFFFF0000u); }

// Round-to-nearest-even fp32 -> bf16 bits; NaN stays NaN (quiet).
__device__ __forceinline__ uint32_t f32_to_bf16_bits(float f) {
    uint32_t u = as_u32(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return ((u >> 16) | 0x40u) & 0xFFFFu;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_bits(lo) | (f32_to_bf16_bits(hi) << 16);
}

// E8M0 scale byte of a block whose largest |x| has fp32 bits amax (sign
// cleared, finite): floor(log2 amax) - 2 clamped below at -127, plus 127.
// For a normal amax with biased exponent E that is E - 2; every amax below
// 2^-125 (subnormals and zero included) clamps to byte 0.  Non-finite blocks
// are handled by the caller (byte 0xFF).
__device__ __forceinline__ uint32_t e8m0_from_amax(uint32_t amax_bits) {
    int E = (int)(amax_bits >> 23);
    return (uint32_t)(E > 2 ? E - 2 : 0);
}

// 2^(byte-127) as an fp32 (byte 0 -> the subnormal 2^-127), the scale operand
// of the gfx950 scaled conversion instructions.
__device__ __forceinline__ float e8m0_scale_f32(uint32_t byte) {
    return as_f32(byte ? (byte << 23) : 0x00400000u);
}

// 2^(127-byte) as an fp32 (exact for byte in [0, 252], the bytes a finite
// block produces).
__device__ __forceinline__ float e8m0_inv_scale_f32(uint32_t byte) {
    return as_f32((254u - byte) << 23);
}

// ---------------------------------------------------------------------------
// Cross-lane max within aligned groups of G lanes (G = 2, 4, 8, 16), through
// DPP lane permutes inside a 16-lane row: quad_perm swaps for the first two
// steps, then the half-row and row mirrors (after the earlier steps every lane
// of a quad / half-row holds the same value, so mirroring pairs the groups).
// ---------------------------------------------------------------------------
template <int G>
__device__ __forceinline__ uint32_t group_max_u32(uint32_t v) {
    if (G >= 2) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0xB1, 0xF, 0xF, false));
    if (G >= 4) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x4E, 0xF, 0xF, false));
    if (G >= 8) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x141, 0xF, 0xF, false));
    if (G >= 16) v = max(v, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)v, 0x140, 0xF, 0xF, false));
    return v;
}

// ---------------------------------------------------------------------------
// Philox4x32 (Salmon, Moraes, Dror, Shaw, SC'11), 10 rounds: counter words
// c0..c3, key words k0, k1.  Each round multiplies c0 and c2 by the Philox
// multipliers, keeps both halves of the 64-bit products and mixes them with
// c1, c3 and the round key; the key advances by the Weyl constants between
// rounds.
// ---------------------------------------------------------------------------
struct Philox4 {
    uint32_t v[4];
};

__device__ __forceinline__ Philox4 philox4x32_10(uint32_t c0, uint32_t c1, uint32_t c2,
                                                 uint32_t c3, uint32_t k0, uint32_t k1) {
#pragma unroll
    for (int r = 0; r < 10; ++r) {
        uint64_t p0 = (uint64_t)0xD2511F53u * c0;
        uint64_t p1 = (uint64_t)0xCD9E8D57u * c2;
        // three-input XORs in one v_bitop3_b32 each (truth table 0x96)
        uint32_t n0 = __builtin_amdgcn_bitop3_b32((uint32_t)(p1 >> 32), c1, k0, 0x96);
        uint32_t n2 = __builtin_amdgcn_bitop3_b32((uint32_t)(p0 >> 32), c3, k1, 0x96);
        c1 = (uint32_t)p1;
        c3 = (uint32_t)p0;
        c0 = n0;
        c2 = n2;
        k0 += 0x9E3779B9u;
        k1 += 0xBB67AE85u;
    }
    Philox4 o;
    o.v[0] = c0;
    o.v[1] = c1;
    o.v[2] = c2;
    o.v[3] = c3;
    return o;
}

// Words of the 16-bit lanes S .. S+7 of the 16-lane stream a, b (lane q is
// half q & 1 of word q >> 1), two lanes per word, low half first.
template <int S>
__device__ __forceinline__ void sr_lanes_from(const Philox4& a, const Philox4& b, uint32_t w[4]) {
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int q0 = S + 2 * k, q1 = S + 2 * k + 1;
        const uint32_t x0 = q0 < 8 ? a.v[(q0 >> 1) & 3] : b.v[((q0 - 8) >> 1) & 3];
        const uint32_t x1 = q1 < 8 ? a.v[(q1 >> 1) & 3] : b.v[((q1 - 8) >> 1) & 3];
        w[k] = ((x0 >> (16 * (q0 & 1))) & 0xFFFFu) | (((x1 >> (16 * (q1 & 1))) & 0xFFFFu) << 16);
    }
}

// Random words for the 8 consecutive logical positions p0 .. p0+7:
// position p uses half (p & 1) of word ((p & 7) >> 1) of the Philox output
// for counter p >> 3 (64-bit, in words 0..1; words 2..3 zero), key = seed.
// w[k] receives the 16-bit lanes of positions p0 + 2k (low half) and
// p0 + 2k + 1 (high half); aligned p0 (the common case) is one call.
__device__ __forceinline__ void sr_words8(uint64_t p0, uint32_t k0, uint32_t k1, uint32_t w[4]) {
    const uint64_t n = p0 >> 3;
    const uint32_t s = (uint32_t)(p0 & 7);
    const Philox4 a = philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), 0u, 0u, k0, k1);
    if (s == 0) {
#pragma unroll
        for (int k = 0; k < 4; ++k) w[k] = a.v[k];
        return;
    }
    const uint64_t n1 = n + 1;
    const Philox4 b = philox4x32_10((uint32_t)n1, (uint32_t)(n1 >> 32), 0u, 0u, k0, k1);
    switch (s) {  // static lane indexing keeps everything in registers
        case 1: sr_lanes_from<1>(a, b, w); break;
        case 2: sr_lanes_from<2>(a, b, w); break;
        case 3: sr_lanes_from<3>(a, b, w); break;
        case 4: sr_lanes_from<4>(a, b, w); break;
        case 5: sr_lanes_from<5>(a, b, w); break;
        case 6: sr_lanes_from<6>(a, b, w); break;
        default: sr_lanes_from<7>(a, b, w); break;
    }
}

// Stochastic rounding to E2M1 with 16 random bits u per element, as gfx950's
// v_cvt_scalef32_sr_pk_fp4_f32 performs it: for m = |x| / scale below 6 the
// fraction of m between its two neighbouring grid values is truncated to 22
// bits, the instruction's 22-bit random field is added, and a carry rounds
// up; m >= 6 gives 6.  With u placed at the top of that field (the field's
// low 6 bits zero) this is exactly: round up iff u + floor(frac * 2^16) >=
// 2^16.  The field of the first element of a pair is bits 31..10 of the
// random word (word = u << 16), that of the second bits 30..9 (u << 15);
// the two overlap, so each element of a pair gets its own conversion.
//
// The instruction writes only the selected byte of its destination and the
// compiler does not tie the builtin's `old` operand to it, so only byte 0 of
// a result is used and the rest is masked off.
//
// Code byte of the pair (x0, x1) sharing scale sc: x0 with random word
// seed0 = u0 << 16 (low nibble of the first conversion), x1 with
// seed1 = u1 << 15 (high nibble of the second).
__device__ __forceinline__ uint32_t sr_pair(float x0, float x1, float sc, uint32_t seed0,
                                            uint32_t seed1) {
    const uint32_t a = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, (f32x2_t){x0, x1}, seed0, sc, 0);
    const uint32_t b = __builtin_amdgcn_cvt_scalef32_sr_pk_fp4_f32(0u, (f32x2_t){x0, x1}, seed1, sc, 0);
    return (a & 0x0Fu) | (b & 0xF0u);
}

// Random words of the pair whose lanes are the low (first element) and high
// (second element) halves of one Philox word w.
__device__ __forceinline__ uint32_t sr_seed_lo(uint32_t w) { return w << 16; }
__device__ __forceinline__ uint32_t sr_seed_hi(uint32_t w) { return (w >> 1) & 0x7FFF8000u; }

// 8 values sharing one scale (a row-direction chunk) whose 16-bit lanes are
// the halves of w[0..3] (see sr_words8), packed two codes per byte.
__device__ __forceinline__ uint32_t sr_pack8(const float x[8], float sc, const uint32_t w[4]) {
    uint32_t r = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k)
        r |= sr_pair(x[2 * k], x[2 * k + 1], sc, sr_seed_lo(w[k]), sr_seed_hi(w[k])) << (8 * k);
    return r;
}

// DGE derivative d(x) for one element with inverse block scale inv (the
// MSRA FP4-training summary page, sec. 二): with m = |x| inv and
// E = max(biased exponent(m), 127), q = m 2^(128 - E) puts every E2M1
// interval at unit width, u = 2 (q - floor(q)) - 1 exactly, and
// d = min((1/k) |u|^(1/k - 1), clamp_max) via the hardware log2/exp2;
// m > 6 (saturated) gives 1.  Shared by the gradient-estimator kernels and the
// GEMM epilogue that applies it, so both give the same bits.
struct DgeParams {
    float invk, p, clamp_max;
    int k_one;
};

__device__ __forceinline__ float dge_factor(float x, float inv, DgeParams P) {
    const float m = fabsf(x) * inv;
    if (m > 6.0f) return 1.0f;
    const uint32_t E = max(as_u32(m) >> 23, 127u);
    const float q = m * as_f32((255u - E) << 23);
    const float u = 2.0f * (q - floorf(q)) - 1.0f;
    float d;
    if (P.k_one) {
        d = 1.0f;
    } else {
        d = P.invk * __builtin_amdgcn_exp2f(P.p * __builtin_amdgcn_logf(fabsf(u)));
    }
    return fminf(d, P.clamp_max);
}

}  // namespace fp4q
