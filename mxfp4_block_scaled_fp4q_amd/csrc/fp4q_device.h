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
        uint32_t n0 = (uint32_t)(p1 >> 32) ^ c1 ^ k0;
        uint32_t n2 = (uint32_t)(p0 >> 32) ^ c3 ^ k1;
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

// 16-bit random lanes for the 8 consecutive logical positions p0 .. p0+7:
// position p uses half (p & 1) of word ((p & 7) >> 1) of the Philox output
// for counter p >> 3 (64-bit, in words 0..1; words 2..3 zero), key = seed.
// u[j] receives the bits of position p0 + j.
__device__ __forceinline__ void sr_bits8(uint64_t p0, uint32_t k0, uint32_t k1, uint32_t u[8]) {
    uint64_t n = p0 >> 3;
    uint32_t s = (uint32_t)(p0 & 7);
    Philox4 a = philox4x32_10((uint32_t)n, (uint32_t)(n >> 32), 0u, 0u, k0, k1);
    if (s == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) u[j] = (a.v[j >> 1] >> (16 * (j & 1))) & 0xFFFFu;
    } else {
        uint64_t n1 = n + 1;
        Philox4 b = philox4x32_10((uint32_t)n1, (uint32_t)(n1 >> 32), 0u, 0u, k0, k1);
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            uint32_t q = s + (uint32_t)j;
            uint32_t w = (q < 8) ? a.v[(q >> 1) & 3] : b.v[((q - 8) >> 1) & 3];
            u[j] = (w >> (16 * (q & 1))) & 0xFFFFu;
        }
    }
}

// Stochastic rounding of one element x (finite, in a block with inverse scale
// inv = 2^-e) to a 4-bit E2M1 code, with 16 random bits u:
//   m = |x| / 2^e;  lo, hi = neighbouring grid values;  round up iff
//   u < (m - lo) / (hi - lo) * 2^16;  m >= 6 gives 6.
// Working variable q = m * 2^(128 - E), E = max(biased exponent of m, 127),
// puts every grid interval at unit width: q in [0, 2) for m < 1 (step 0.5),
// q in [2, 4) for m in [1, 8) (steps 0.5, 1, 2); the code is
// 2 (E - 127) + floor(q) (+1 on round-up), capped at 7.  All of this is exact
// in fp32 while m is normal.  When m is below the normal range (only possible
// for a nonzero x far below its block max) the exact threshold is under 1, so
// the decision is "round up iff u == 0 and x != 0": T is raised to 0.5 there.
__device__ __forceinline__ uint32_t sr_code(float x, float inv, uint32_t u) {
    uint32_t xb = as_u32(x);
    float m = fabsf(x) * inv;
    uint32_t mb = as_u32(m);
    uint32_t E = max(mb >> 23, 127u);
    float q = m * as_f32((255u - E) << 23);
    float fl = floorf(q);
    float T = (q - fl) * 65536.0f;
    if ((xb & 0x7FFFFFFFu) != 0u && fl == 0.0f) T = fmaxf(T, 0.5f);
    uint32_t up = ((float)u < T) ? 1u : 0u;
    uint32_t code = 2u * (E - 127u) + (uint32_t)fl + up;
    code = min(code, 7u);
    return code | ((xb >> 28) & 8u);
}

}  // namespace fp4q
