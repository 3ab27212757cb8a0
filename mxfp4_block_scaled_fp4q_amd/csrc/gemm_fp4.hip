// FP4 x FP4 GEMM with per-block E8M0 scales on CDNA4 scaled MFMA.
//
//   C[i, j] (+)= sum_k deq(A[i, k]) * deq(B[j, k]),  fp32 accumulation
//
// The FP4 GEMMs carry the bulk of the layer's compute (MSRA FP4-training
// summary page, sec. 四: matrix multiplies are over 95% of a Transformer's
// work and are the part moved to FP4); the pages' own kernels are FP8
// emulation on H100 (same page, sec. 五) and Blackwell tensor cores, so this
// is a gfx950 design, not a port: v_mfma_scale_f32_32x32x64_f8f6f4 with both
// operands in E2M1 applies one E8M0 byte per 32 K-elements of each row of A
// and of B inside the instruction.
//
// Operand layout that the instruction expects (pinned on the device with
// random operands): lane l supplies row (l % 32) of the 32x64 A tile, K
// elements [32 (l / 32), 32 (l / 32) + 32) as 16 consecutive bytes -- exactly
// 16 contiguous bytes of a K-major code row, low nibble first -- plus the
// scale byte of that row and 32-element K block; B likewise by column.  The
// 32x32 fp32 result sits in 16 registers: register r of lane l holds row
// 8 (r / 4) + 4 (l / 32) + r % 4, column l % 32.
//
// Tiling: a workgroup of 8 waves (2 along M x 4 along N) computes a 256 x 256
// tile of C, each wave 128 x 64 as 4 x 2 MFMA tiles (128 accumulator
// registers), or a 128 x 384 tile, each wave 64 x 96 as 2 x 3 MFMA tiles,
// where the latter saves a whole round of tiles (it is 3/4 of the work per
// tile but measured 1.45x slower per flop, so the 256 x 256 tile is the
// default).  Two waves share every SIMD, so one wave's MFMAs run while the
// other waits on LDS or the barrier.  The K loop steps 64 bytes per operand
// row (128 FP4 or 32 bf16 elements).
//
// Operands go global -> LDS directly (buffer loads with the LDS bit, so no
// registers are spent on staging) through a 4-stage ring, issued three
// steps ahead of their use.  Each code load instruction fills one 1 KB
// region of 16 rows x 64 bytes in lane order; lane 4j + p fetches chunk
// p ^ ((j / 4) % 4) of row j, so the four lanes of a row read its 64 bytes
// together while the rotated chunk order makes the MFMA-side 16-byte reads
// (lane = row) free of bank conflicts.  Scale bytes are fetched in groups of
// 8 K steps (32 contiguous bytes per row, eight lanes per row) into a
// double-buffered LDS ring, a group being loaded during the first half of
// the group before it; the cost of a load instruction on this path grows
// with the number of distinct rows it touches, so this is 8x cheaper than a
// 4-byte word per row per step.  Rows past M or N read as zero (per-tile
// buffer ranges).  The epilogue stages each wave's tile in LDS so every lane
// writes 16 contiguous bytes.  Workgroups are remapped so that consecutive
// tiles of a grouped (4 tile-rows) order run on the same XCD and share its
// L2.  Where there are more 256 x 256 tiles than compute units and K is a
// multiple of 1024, a persistent form runs instead (one workgroup per compute
// unit walking its tiles with the operand ring running on across tiles, the
// workgroups with a tile fewer starting a little late; see
// gemm_fp4_persistent_kernel).
#include <algorithm>
#include <cstdlib>
#include <cstring>
#include <type_traits>

#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
// Native 4 x 32-bit vectors (HIP's uint4 is a class with unions, which the
// compiler does not always split into registers).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;

static constexpr int BKB = 64;                  // operand bytes per row per K step
static constexpr int REGION = 1024;             // 16 rows x 64 bytes
static constexpr int STAGE = 32 * REGION;       // one K step of A and B codes
static constexpr int SROW = 32;                 // LDS bytes per scale row per group
static constexpr int SCALE_BUF = 512 * SROW;    // A rows, then B rows
// K steps per scale group: 8 (32 scale bytes per row) when every scale row
// starts on a 4-byte boundary (K % 128 == 0); 4 when K % 128 == 64, where the
// rows are only 2-byte aligned and are fetched with 2-byte loads, each of
// which fills a whole LDS dword (low half data, high half zero), so a group
// of 16 data bytes still takes 32 bytes of LDS per row.
template <int TAIL> struct Groups {
    static constexpr int SG = TAIL ? 4 : 8;
    static constexpr int SGB = 4 * SG;          // scale bytes per row per group in memory
};
static constexpr int GROUP_M = 4;
static constexpr int BUF_FLAGS = 0x00020000;    // buffer resource word 3: raw 32-bit data

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14; expcnt 6:4 and lgkmcnt 11:8 at maximum).
#define FP4Q_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x0F70)

// Tile configurations: eight waves, two along M and four along N, each
// owning TM x TN MFMA tiles of 32 x 32.
//   CFG 0: 256 x 256 tile, 128 x 64 per wave (4 x 2 MFMA tiles);
//   CFG 1: 128 x 384 tile,  64 x 96 per wave (2 x 3 MFMA tiles), for shapes
//          whose 256 x 256 tiles would leave part of the chip idle in the
//          last round (three of its tiles cover the area of four of those).
// Both stage 512 operand rows (32 KB) per K step and 512 scale rows.
template <int CFG>
struct Layout {
    static constexpr int WAVES = 8, THREADS = 64 * WAVES;
    static constexpr int WM = 2, WN = 4;
    static constexpr int TM = CFG == 0 ? 4 : 2;  // 32-row MFMA tiles per wave
    static constexpr int TN = CFG == 0 ? 2 : 3;  // 32-column MFMA tiles per wave
    static constexpr int WROWS = 32 * TM, WCOLS = 32 * TN;
    static constexpr int BM = WM * WROWS, BN = WN * WCOLS;
    static constexpr int RA = BM / 16, RB = BN / 16;  // 1 KB code regions per step
    static constexpr int RPW_A = RA / WAVES, RPW_B = RB / WAVES;
    static constexpr int RPW = RPW_A > RPW_B ? RPW_A : RPW_B;
    static constexpr int OFF_B = RA * REGION;         // B codes within a stage
    static constexpr int SROWS = 512 / WAVES;         // scale rows fetched per wave
    static constexpr int SPIECES = SROWS / 8;         // 8-row scale pieces per wave per group
    static constexpr int A_SWAVES = BM / SROWS;       // waves fetching A scale rows
    static_assert(RA % WAVES == 0 && RB % WAVES == 0, "code regions divide among the waves");
    static_assert((RA + RB) * REGION == STAGE, "one 32 KB stage per K step");
    static_assert(BM + BN == WAVES * SROWS, "the waves fetch all scale rows");
    static_assert(SPIECES % 4 == 0, "scale pieces spread over four steps");
};

// 16-byte slot of chunk c (bytes 16c .. 16c+15 of the step) of row j within
// a 16-row region.
__device__ __forceinline__ int region_slot(int j, int c) { return 4 * j + (c ^ ((j >> 2) & 3)); }

// Load sources: buffer resources whose ranges end at the operand's last row
// inside this tile (rows past M or N read as zero), 32-bit per-lane offsets
// (they alone decide whether a row is in range), and the scalar byte offset
// of the current K step.
template <int CFG>
struct Src {
    __amdgpu_buffer_rsrc_t ra, rb, rsc;  // rsc: scales of this wave's pieces (A or B)
    uint32_t vrow[Layout<CFG>::RPW];     // region q of A and of B share the row offsets
    uint32_t vsc[4];  // scale piece offsets, by piece index % 4 (word swizzle)
    int soff;
};

// Direct-to-LDS loads of the K step the sources point at into `stage`; the
// sources then advance to the next step if `advance` (past the end of K the
// last step is re-issued into a stage nobody reads again, so every step
// issues the same number of loads and the waits are compile-time).
template <int CFG, int BF16OPS>
__device__ __forceinline__ void issue_codes(Src<CFG>& src, uint8_t* stage, int wave,
                                            bool advance) {
    using L = Layout<CFG>;
#pragma unroll
    for (int q = 0; q < L::RPW; ++q) {
        const int rho = q * L::WAVES + wave;
        if (q < L::RPW_A)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(src.ra, (lds_ptr_t)(stage + rho * REGION), 16,
                                                     src.vrow[q], src.soff, 0, 0);
        if (q < L::RPW_B)
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                src.rb, (lds_ptr_t)(stage + L::OFF_B + rho * REGION), 16, src.vrow[q], src.soff, 0,
                0);
    }
    src.soff += advance ? BKB : 0;
}

// Scale piece P (0 .. SPIECES-1) of this wave for group g: combined rows
// wave*SROWS + P*8 .. +7 (A rows 0..BM-1, then B rows), 32 LDS bytes each.
// Whole words (TAIL = 0): lane 8j + pos loads word pos ^ (P % 4) of the
// piece's row j, so that in LDS word s of row R sits at R*32 + 4 (s ^ ((R / 8)
// % 4)) (SROWS / 8 is a multiple of 4).  Half words (TAIL = 1): lane 8j + pos
// loads half (pos % 2) of word (pos / 2) ^ (P % 4) into LDS dword pos of row
// j, so that word s of row R is the low halves of the dwords at R*32 +
// 8 (s ^ ((R / 8) % 4)) and the next one.  The group offset is part of the
// per-lane offset so the range check covers it.
template <int CFG, int P, int TAIL>
__device__ __forceinline__ void issue_scale_piece(const Src<CFG>& src, uint8_t* sbuf, int wave,
                                                  int kscale, int g) {
    // the uniform part as one scalar, so that the compiler does not keep a
    // hoisted per-piece vector offset live across the K loop
    uint32_t soff = (uint32_t)(P * 8 * kscale + g * Groups<TAIL>::SGB);
    asm volatile("" : "+s"(soff));
    const uint32_t voff = src.vsc[P & 3] + soff;
    lds_ptr_t dst = (lds_ptr_t)(sbuf + (wave * Layout<CFG>::SROWS + P * 8) * SROW);
    if constexpr (TAIL)
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.rsc, dst, 2, voff, 0, 0, 0);
    else
        __builtin_amdgcn_raw_ptr_buffer_load_lds(src.rsc, dst, 4, voff, 0, 0, 0);
}

// Pieces P0 .. P0+N-1.
template <int CFG, int P0, int N, int TAIL>
__device__ __forceinline__ void issue_scale_pieces(const Src<CFG>& src, uint8_t* sbuf, int wave,
                                                   int kscale, int g) {
    if constexpr (N > 0) {
        issue_scale_piece<CFG, P0, TAIL>(src, sbuf, wave, kscale, g);
        issue_scale_pieces<CFG, P0 + 1, N - 1, TAIL>(src, sbuf, wave, kscale, g);
    }
}

template <int CFG>
struct Frags {
    u32x4 a[Layout<CFG>::TM], b[Layout<CFG>::TN];
};

// This wave's A and B fragments of one half of a staged step; `off` is this
// lane's offset within a 32-row group for that half (row lane % 32, chunk
// 2 kk + lane / 32).
template <int CFG>
__device__ __forceinline__ void read_frags(const uint8_t* base, int off, int wm, int wn,
                                           Frags<CFG>& F) {
    using L = Layout<CFG>;
#pragma unroll
    for (int i = 0; i < L::TM; ++i)
        F.a[i] = *(const u32x4*)(base + (wm * L::TM + i) * 2 * REGION + off);
#pragma unroll
    for (int j = 0; j < L::TN; ++j)
        F.b[j] = *(const u32x4*)(base + L::OFF_B + (wn * L::TN + j) * 2 * REGION + off);
}

// Scale words (4 K blocks of 32 elements each) of step word s of a group
// for this lane's MFMA rows (A) and columns (B); `sx` is this lane's
// swizzled byte offset of that word: 4 (s ^ ((lane % 32) / 8 % 4)) for whole
// words, 8 (s ^ ...) for the half-word layout (TAIL), whose two dwords carry
// the word's low and high halves.
template <int CFG, int TAIL>
__device__ __forceinline__ uint32_t scale_word(const uint8_t* p) {
    if constexpr (TAIL) {
        const uint2 d = *(const uint2*)p;
        return (d.x & 0xFFFFu) | (d.y << 16);
    } else {
        return *(const uint32_t*)p;
    }
}

template <int CFG, int TAIL>
__device__ __forceinline__ void read_scales(const uint8_t* sbuf, int sx, int wm, int wn, int lane,
                                            uint32_t (&sa)[Layout<CFG>::TM],
                                            uint32_t (&sb)[Layout<CFG>::TN]) {
    using L = Layout<CFG>;
    const int l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < L::TM; ++i)
        sa[i] = scale_word<CFG, TAIL>(sbuf + (wm * L::WROWS + i * 32 + l32) * SROW + sx);
#pragma unroll
    for (int j = 0; j < L::TN; ++j)
        sb[j] = scale_word<CFG, TAIL>(sbuf + (L::BM + wn * L::WCOLS + j * 32 + l32) * SROW + sx);
}

// Shifts raw scale words so that byte 2 kk is the K block of half kk for
// this lane's 32-element K chunk (lanes 32..63 take the odd blocks).
template <int CFG>
__device__ __forceinline__ void shift_scales(const uint32_t (&ra)[Layout<CFG>::TM],
                                             const uint32_t (&rb)[Layout<CFG>::TN], int sh,
                                             uint32_t (&sa)[Layout<CFG>::TM],
                                             uint32_t (&sb)[Layout<CFG>::TN]) {
#pragma unroll
    for (int i = 0; i < Layout<CFG>::TM; ++i) sa[i] = ra[i] >> sh;
#pragma unroll
    for (int j = 0; j < Layout<CFG>::TN; ++j) sb[j] = rb[j] >> sh;
}

// The TM x TN MFMAs of this wave on half KK of a K step.  FP4: the scaled
// MFMA on E2M1 operands (64 K elements per half), its byte select picking
// byte 2 KK of the lane's (pre-shifted) scale words; BF16: plain bf16 MFMAs
// (16 K elements per half, the same 16 bytes per lane).  B is the MFMA's
// first operand, so each accumulator holds the transposed tile: register r
// of lane l is C[row l % 32][column 8 (r / 4) + 4 (l / 32) + r % 4], four
// consecutive columns per register group, which the epilogue stores whole.
template <int CFG, int BF16OPS, int KK>
__device__ __forceinline__ void mfma_half(const Frags<CFG>& F, const uint32_t (&sa)[Layout<CFG>::TM],
                                          const uint32_t (&sb)[Layout<CFG>::TN],
                                          v16f (&acc)[Layout<CFG>::TM][Layout<CFG>::TN]) {
    using L = Layout<CFG>;
    if (BF16OPS) {
#pragma unroll
        for (int i = 0; i < L::TM; ++i)
#pragma unroll
            for (int j = 0; j < L::TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, F.b[j]), __builtin_bit_cast(bf16x8_t, F.a[i]),
                    acc[i][j], 0, 0, 0);
        return;
    }
#pragma unroll
    for (int i = 0; i < L::TM; ++i) {
        const v8i fa = (v8i){(int)F.a[i].x, (int)F.a[i].y, (int)F.a[i].z, (int)F.a[i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < L::TN; ++j) {
            const v8i fb =
                (v8i){(int)F.b[j].x, (int)F.b[j].y, (int)F.b[j].z, (int)F.b[j].w, 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fb, fa, acc[i][j], 4, 4, 2 * KK, (int)sb[j], 2 * KK, (int)sa[i]);
        }
    }
}

// The LDS ring stages and scale buffers: separate objects, so the compiler
// sees that loads in flight into one stage and reads of another do not
// alias; the epilogue reuses the stages.
__shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
__shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
__shared__ __attribute__((aligned(16))) uint8_t st2[STAGE];
__shared__ __attribute__((aligned(16))) uint8_t st3[STAGE];
__shared__ __attribute__((aligned(16))) uint8_t sc0[SCALE_BUF];
__shared__ __attribute__((aligned(16))) uint8_t sc1[SCALE_BUF];

// One K loop of the workgroup's tile over operands ac / bc (K-major rows, K
// elements deep; FP4 with scales as, bs, or bf16 without), accumulating into
// acc.  Leaves no loads in flight; the caller synchronises before the stages
// are reused.  TAIL (FP4 only, K % 128 == 64): the last K step holds one half
// (its second half's MFMAs are skipped; what its loads fetch past the row is
// never used) and the scale rows, only 2-byte aligned, go through the
// half-word layout in groups of 4 steps.
template <int CFG, int BF16OPS, int TAIL>
__device__ __forceinline__ void gemm_kloop(v16f (&acc)[Layout<CFG>::TM][Layout<CFG>::TN],
                                           const uint8_t* __restrict__ ac,
                                           const uint8_t* __restrict__ as,
                                           const uint8_t* __restrict__ bc,
                                           const uint8_t* __restrict__ bs, int K, int M, int N,
                                           int m0, int n0, int wave, int lane, int wm, int wn,
                                           int half, int l32, int off0, int off1, int sxor) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot instantiate buffer resources
    using L = Layout<CFG>;
    constexpr int TM = L::TM, TN = L::TN;
    static_assert(!(TAIL && BF16OPS), "bf16 K loops are whole steps");
    constexpr int SG = Groups<TAIL>::SG;
    // bytes per operand row (< 2^23, checked by the caller); each K step
    // consumes 64 of them (the last one 32 with TAIL)
    const int kbytes = BF16OPS ? K * 2 : K / 2;
    const int kscale = K / 32;
    const int ksteps = (kbytes + BKB - 1) / BKB;

    Src<CFG> src;
    {
        const int rows_a = min(M - m0, L::BM), rows_b = min(N - n0, L::BN);
        src.ra = __builtin_amdgcn_make_buffer_rsrc((void*)(ac + (int64_t)m0 * kbytes), (short)0,
                                                   rows_a * kbytes, BUF_FLAGS);
        src.rb = __builtin_amdgcn_make_buffer_rsrc((void*)(bc + (int64_t)n0 * kbytes), (short)0,
                                                   rows_b * kbytes, BUF_FLAGS);
        // lane 4j + p of a region loads chunk p ^ ((j / 4) % 4) of row j
        const int j = lane >> 2;
        const int c = (lane & 3) ^ ((j >> 2) & 3);
#pragma unroll
        for (int q = 0; q < L::RPW; ++q)
            src.vrow[q] = (uint32_t)(((q * L::WAVES + wave) * 16 + j) * kbytes + c * 16);
        // waves 0 .. A_SWAVES-1 fetch A scale rows, the others B
        constexpr int HW = L::A_SWAVES;
        src.rsc = wave < HW ? __builtin_amdgcn_make_buffer_rsrc((void*)(as + (int64_t)m0 * kscale),
                                                                (short)0, rows_a * kscale, BUF_FLAGS)
                            : __builtin_amdgcn_make_buffer_rsrc((void*)(bs + (int64_t)n0 * kscale),
                                                                (short)0, rows_b * kscale, BUF_FLAGS);
        const int sbase = ((wave < HW ? wave : wave - HW) * L::SROWS + (lane >> 3)) * kscale;
#pragma unroll
        for (int q = 0; q < 4; ++q)
            src.vsc[q] = TAIL ? (uint32_t)(sbase + ((((lane & 7) >> 1) ^ q) << 2) + ((lane & 1) << 1))
                              : (uint32_t)(sbase + (((lane & 7) ^ q) << 2));
        src.soff = 0;
    }
    Frags<CFG> FA, FB;
    // sa/sb: shifted scale words of the step being computed; ra/rb: raw
    // words of the next step, read after the barrier that publishes it.
    uint32_t sa[TM], ra[TM], sb[TN], rb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = ra[i] = 0;
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[j] = rb[j] = 0;
    const int sh = 8 * half;

    // Software pipeline over K steps t with a 4-stage code ring: step t
    // issues the code loads of step t + 3 into the stage step t - 1 used
    // (every wave finished reading it before the previous barrier), and, in
    // the first half of each 8-step scale group, two scale pieces of the next
    // group into the other scale buffer (its previous group ended before);
    // with TAIL's 4-step groups, all eight pieces in the group's first step
    // (so that they have landed by the wait at the end of its last step).  Each
    // step computes two halves (K bytes 0..31 and 32..63 of the step); order
    // within a step, fenced against the compiler's scheduler:
    //   1. shift the step's scale words; read the fragments of (t, 1); issue
    //      loads;
    //   2. MFMAs of (t, 0), whose fragments were read during step t - 1;
    //   3. wait for this wave's loads of step t + 1 (later loads stay in
    //      flight) and its LDS reads, then one workgroup barrier;
    //   4. read the scales and (t + 1, 0) fragments; MFMAs of (t, 1).
    // The loop is unrolled by 16 steps (two or four scale groups, four turns
    // of the ring), so every load count, wait and LDS buffer is a
    // compile-time constant.
    constexpr int LC = L::RPW_A + L::RPW_B;  // code loads per wave per step
    // loads issued after the code loads of step t + 1, at the end of step t
    // with t % 8 == p: those of steps t - 1 and t plus the scale pieces
    // issued after the code loads in step t - 2
#define FP4Q_PIECES(p)                                                              \
    (BF16OPS ? 0 : TAIL ? ((((p) & 3) == 0) ? L::SPIECES : 0)                          \
                        : ((((p) & 7) >= 4) ? 0 : L::SPIECES / 4))
#define FP4Q_BEHIND(p) (FP4Q_PIECES((p) + 6) + LC + FP4Q_PIECES((p) + 7) + LC + FP4Q_PIECES(p))
    if (!BF16OPS) issue_scale_pieces<CFG, 0, L::SPIECES, TAIL>(src, sc0, wave, kscale, 0);
    issue_codes<CFG, BF16OPS>(src, st0, wave, 1 < ksteps);
    issue_codes<CFG, BF16OPS>(src, st1, wave, 2 < ksteps);
    issue_codes<CFG, BF16OPS>(src, st2, wave, 3 < ksteps);
    FP4Q_WAIT_VMCNT(2 * LC);
    __builtin_amdgcn_s_barrier();
    if (!BF16OPS) read_scales<CFG, TAIL>(sc0, TAIL ? sxor << 3 : sxor << 2, wm, wn, lane, ra, rb);
    read_frags<CFG>(st0, off0, wm, wn, FA);

// One K step t = kt + P (P = t % 16, compile-time; its position in its
// scale group is P % SG).  The scale buffer of step P's group and of the
// next group alternate with the group's parity.  The final step's reads of
// a next step are harmless (in-bounds, unused), so no step is special, except
// that with TAIL the last step's second half has no data.
#define FP4Q_SCUR(P) ((((P) / SG) & 1) ? sc1 : sc0)
#define FP4Q_SNXT(P) ((((P) / SG) & 1) ? sc0 : sc1)
#define FP4Q_GEMM_STEP(P, CUR, NEXT1, NEXTL)                                         \
    do {                                                                             \
        const int t_ = kt + (P);                                                     \
        __builtin_amdgcn_sched_barrier(0);                                           \
        if (!BF16OPS) shift_scales<CFG>(ra, rb, sh, sa, sb);                          \
        read_frags<CFG>(CUR, off1, wm, wn, FB);                                       \
        issue_codes<CFG, BF16OPS>(src, NEXTL, wave, t_ + 4 < ksteps);                 \
        if (FP4Q_PIECES(P))                                                          \
            issue_scale_pieces<CFG, TAIL ? 0 : ((P) & 3) * (L::SPIECES / 4),             \
                               FP4Q_PIECES(P), TAIL>(src, FP4Q_SNXT(P), wave, kscale,      \
                                                     t_ / SG + 1);                       \
        __builtin_amdgcn_sched_barrier(0);                                           \
        mfma_half<CFG, BF16OPS, 0>(FA, sa, sb, acc);                                  \
        __builtin_amdgcn_sched_barrier(0);                                           \
        FP4Q_WAIT_VMCNT(FP4Q_BEHIND(P));                                             \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                          \
        __builtin_amdgcn_s_barrier();                                                \
        __builtin_amdgcn_sched_barrier(0);                                           \
        if (!BF16OPS)                                                                \
            read_scales<CFG, TAIL>(((P) % SG) == SG - 1 ? FP4Q_SNXT(P) : FP4Q_SCUR(P),       \
                                   TAIL ? (((P) + 1) & 3 ^ sxor) << 3                       \
                                        : (((P) + 1) & 7 ^ sxor) << 2,                      \
                                   wm, wn, lane, ra, rb);                                \
        read_frags<CFG>(NEXT1, off0, wm, wn, FA);                                     \
        if (!TAIL || t_ != ksteps - 1) mfma_half<CFG, BF16OPS, 1>(FB, sa, sb, acc);   \
    } while (0)

// Eight steps starting at t = kt + O (two turns of the code ring); GUARD(P)
// says whether step kt + P exists (compile-time true in full turns).
#define FP4Q_GEMM_GROUP(O, GUARD)                                                    \
    do {                                                                             \
        if (GUARD(O + 0)) FP4Q_GEMM_STEP(O + 0, st0, st1, st3);                       \
        if (GUARD(O + 1)) FP4Q_GEMM_STEP(O + 1, st1, st2, st0);                       \
        if (GUARD(O + 2)) FP4Q_GEMM_STEP(O + 2, st2, st3, st1);                       \
        if (GUARD(O + 3)) FP4Q_GEMM_STEP(O + 3, st3, st0, st2);                       \
        if (GUARD(O + 4)) FP4Q_GEMM_STEP(O + 4, st0, st1, st3);                       \
        if (GUARD(O + 5)) FP4Q_GEMM_STEP(O + 5, st1, st2, st0);                       \
        if (GUARD(O + 6)) FP4Q_GEMM_STEP(O + 6, st2, st3, st1);                       \
        if (GUARD(O + 7)) FP4Q_GEMM_STEP(O + 7, st3, st0, st2);                       \
    } while (0)
#define FP4Q_ALL(P) true
#define FP4Q_EXISTS(P) (kt + (P) < ksteps)

    // Step t uses code stage t % 4 and scale buffer (t / SG) % 2; a turn of
    // the loop covers 16 steps so every buffer is named at compile time (the
    // compiler then sees that scale reads and the loads in flight touch
    // different LDS objects).
    int kt = 0;
    for (; kt + 16 <= ksteps; kt += 16) {
        FP4Q_GEMM_GROUP(0, FP4Q_ALL);
        FP4Q_GEMM_GROUP(8, FP4Q_ALL);
    }
    if (kt < ksteps) {
        FP4Q_GEMM_GROUP(0, FP4Q_EXISTS);
        FP4Q_GEMM_GROUP(8, FP4Q_EXISTS);
    }
#undef FP4Q_GEMM_GROUP
#undef FP4Q_GEMM_STEP
#undef FP4Q_SCUR
#undef FP4Q_SNXT
#undef FP4Q_ALL
#undef FP4Q_EXISTS
#undef FP4Q_PIECES
#undef FP4Q_BEHIND
    FP4Q_WAIT_VMCNT(0);  // the re-issued loads past the end of K have landed
#endif
}

// OPS: 0 = FP4 operands; 1 = bf16 operands (ac, bc hold bf16 rows, no
// scales; with ACCUM, kp is the size of the first round of workgroups, see
// below); 2 = FP4 over K, then bf16 over the kp-deep operands ha, hb into
// the same accumulators (the single-kernel hot-channel compensation).
// EPI = 1 (fp32 C, 256 x 256 tiles, M % 32 == 0): C is multiplied in the
// epilogue by the DGE derivative of ex [M, N] (bf16, dense) with ex's column
// blocks of 32 rows -- the weight gradient's estimator applied where the
// weight gradient is produced.
// EPI = 2 (bf16 C, 256 x 256 tiles, N % 32 == 0): the bf16 C is also
// quantised (ROW blocks of 32, nearest-even) into qc [M, N/2] and qs
// [M, N/32], as fp4q_quantize would from the stored C; cptr may be null.
// TAIL: K % 128 == 64 (the FP4 K loop ends on a half step; see gemm_kloop).
template <int CFG, int OUT_BF16, int ACCUM, int OPS, int EPI = 0, int TAIL = 0>
__global__ __launch_bounds__(Layout<CFG>::THREADS, 1) void gemm_fp4_kernel(
    int M, int N, int K, const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, void* __restrict__ cptr,
    int64_t ldc, int tiles_m, int tiles_n, const uint8_t* __restrict__ ha,
    const uint8_t* __restrict__ hb, int kp, const uint16_t* __restrict__ ex, DgeParams dp,
    uint8_t* __restrict__ qc, uint8_t* __restrict__ qs) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot instantiate buffer resources
    using L = Layout<CFG>;
    constexpr int TM = L::TM, TN = L::TN;
    static_assert(EPI != 1 || (CFG == 0 && !OUT_BF16 && !ACCUM && OPS == 0),
                  "the DGE epilogue is for fp32 C on 256 x 256 tiles");
    static_assert(EPI != 2 || (CFG == 0 && OUT_BF16 && !ACCUM && OPS == 0),
                  "the quantising epilogue is for bf16 C on 256 x 256 tiles");

    // ---- tile index: XCD-contiguous, then grouped along M ----
    const int nwg = gridDim.x;
    int wg = blockIdx.x;
    {
        const int full = (nwg / 8) * 8;
        if (wg < full) wg = (wg % 8) * (full / 8) + wg / 8;
    }
    const int per_group = GROUP_M * tiles_n;
    const int grp = wg / per_group;
    const int first_m = grp * GROUP_M;
    const int gsize = min(GROUP_M, tiles_m - first_m);
    const int in_grp = wg - grp * per_group;
    const int tm = first_m + in_grp % gsize;
    const int tn = in_grp / gsize;
    const int m0 = tm * L::BM, n0 = tn * L::BN;

    // The accumulating bf16 form (the D-mode residual: C += ..., a read-
    // modify-write of C after each tile's K loop) with several rounds of
    // tiles: kp is the first round's size, and its odd workgroups start about
    // half a tile late (0.5 us per K step + 10 us, a bounded wait on the
    // real-time counter), so that the compute units' read-modify-write phases
    // alternate instead of all hitting memory at once.  13B-shaped residual
    // (461 hot channels): 832 -> 805 us with the gathers, the same bits.
    if (OPS == 1 && ACCUM && (int)blockIdx.x < kp && (blockIdx.x & 1)) {
        const uint64_t until =
            __builtin_amdgcn_s_memrealtime() + (uint64_t)(K / 32) * 50 + 1000;
        while (__builtin_amdgcn_s_memrealtime() < until) __builtin_amdgcn_s_sleep(16);
    }
    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / L::WN, wn = wave % L::WN;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    // this lane's offsets within a 32-row group: row lane % 32, chunk
    // 2 kk + lane / 32
    const int off0 = (l32 >> 4) * REGION + region_slot(l32 & 15, half) * 16;
    const int off1 = (l32 >> 4) * REGION + region_slot(l32 & 15, 2 + half) * 16;
    const int sxor = (l32 >> 3) & 3;  // scale word swizzle of this lane's rows

    v16f acc[TM][TN];
#pragma unroll
    for (int i = 0; i < TM; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;


#define FP4Q_KLOOP(BF, A_, AS_, B_, BS_, KD_)                                              \
    gemm_kloop<CFG, BF, BF ? 0 : TAIL>(acc, A_, AS_, B_, BS_, KD_, M, N, m0, n0, wave, lane, wm, wn, half, l32, \
                       off0, off1, sxor)
    if (OPS == 1) {
        FP4Q_KLOOP(1, ac, as, bc, bs, K);
    } else {
        FP4Q_KLOOP(0, ac, as, bc, bs, K);
        if (OPS == 2 && kp > 0) {
            __syncthreads();  // every wave is done with the stages before they refill
            FP4Q_KLOOP(1, ha, nullptr, hb, nullptr, kp);
        }
    }
#undef FP4Q_KLOOP

    // ---- epilogue: through LDS, so every lane writes 16 contiguous bytes ----
    // Each wave stages its tile 32 rows at a time in a private LDS region
    // (row pitch padded by 16 bytes; a lane writes its four consecutive
    // columns of a row as one 8- or 16-byte access), then reads it back as
    // 16-byte row chunks.
    __syncthreads();  // all waves are done with the operand stages
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int PITCH = L::WCOLS * ESZ + 16;
    constexpr int EREG = 32 * PITCH;
    const int row0 = m0 + wm * L::WROWS;
    const int col0 = n0 + wn * L::WCOLS;
    const bool vec_ok = ((ldc * ESZ) % 16 == 0) && (((uintptr_t)cptr & 15) == 0);
    constexpr int CHUNK_ELEMS = 16 / ESZ;  // elements per 16-byte chunk
    constexpr int LANES_PER_ROW = L::WCOLS / CHUNK_ELEMS;
    constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;  // rows read back per pass
    constexpr int PASSES = (32 + ROWS_PER_PASS - 1) / ROWS_PER_PASS;
    // Accumulating into an fp32 C (C += A B): each 32-row group's C chunks
    // are read ahead of their use, two groups in flight (each group's while
    // the group before it is added and stored), instead of one
    // read-then-write round trip per chunk.  (256 x 256 tiles: 8 chunks per
    // lane per group.  Reading the first group before the K loop would keep
    // 32 more registers live through it, which spills.)  C is read with
    // non-temporal loads, as it is written with non-temporal stores: a
    // stream of C through the L2 evicts the operand rows that the other
    // tiles' K loops read (13B-shaped residual, 461 hot channels: 805 ->
    // 650 us per call with its gathers, the same bits).
    constexpr bool YPF = ACCUM && !OUT_BF16 && EPI == 0 && PASSES <= 8 && L::TM == 4;
    auto c_chunk = [&](int i, int p, int64_t& off) __attribute__((always_inline)) -> bool {
        const int rl = p * ROWS_PER_PASS + lane / LANES_PER_ROW;
        const int row = row0 + i * 32 + rl;
        const int col = col0 + (lane % LANES_PER_ROW) * CHUNK_ELEMS;
        off = (int64_t)row * ldc + col;
        return lane < ROWS_PER_PASS * LANES_PER_ROW && rl < 32 && row < M && vec_ok &&
               col + CHUNK_ELEMS <= N;
    };
    auto c_prefetch = [&](int i, float4 (&y)[YPF ? PASSES : 1]) __attribute__((always_inline)) {
        if constexpr (YPF) {
#pragma unroll
            for (int p = 0; p < PASSES; ++p) {
                int64_t off;
                if (c_chunk(i, p, off))
                    y[p] = __builtin_bit_cast(
                        float4, __builtin_nontemporal_load((const u32x4*)((const float*)cptr + off)));
            }
        }
    };
    float4 ya[YPF ? PASSES : 1], yb[YPF ? PASSES : 1];
    constexpr int PER_STAGE = STAGE / EREG;  // wave regions that fit in one stage
    static_assert(L::WAVES <= 4 * PER_STAGE, "epilogue regions fit in the four stages");
    uint8_t* reg = (wave / PER_STAGE == 0   ? st0
                    : wave / PER_STAGE == 1 ? st1
                    : wave / PER_STAGE == 2 ? st2
                                            : st3) +
                   (wave % PER_STAGE) * EREG;
    // group i of the wave's rows; yv: its C chunks read ahead (YPF)
    auto epi_group = [&](const int i, const float4 (&yv)[YPF ? PASSES : 1])
                         __attribute__((always_inline)) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int g = 0; g < 4; ++g) {
                // row l32 of the pass, columns cl .. cl+3 of the wave's tile
                const int cl = j * 32 + 8 * g + 4 * half;
                uint8_t* dst = reg + l32 * PITCH + cl * ESZ;
                const v16f& a = acc[i][j];
                if (OUT_BF16) {
                    // round-to-nearest-even packs (v_cvt_pk_bf16_f32)
                    const bf16x2_t p0 = {(__bf16)a[4 * g], (__bf16)a[4 * g + 1]};
                    const bf16x2_t p1 = {(__bf16)a[4 * g + 2], (__bf16)a[4 * g + 3]};
                    *(uint2*)dst = make_uint2(__builtin_bit_cast(uint32_t, p0),
                                              __builtin_bit_cast(uint32_t, p1));
                } else {
                    *(u32x4*)dst = (u32x4){as_u32(a[4 * g]), as_u32(a[4 * g + 1]),
                                           as_u32(a[4 * g + 2]), as_u32(a[4 * g + 3])};
                }
            }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
        __builtin_amdgcn_wave_barrier();
        const int rbase = row0 + i * 32;
        // DGE epilogue: these 32 rows are one column block of ex.  Each lane
        // reads ex at the 4 columns and PASSES rows it writes; lanes 16 apart
        // share columns, so two exchanges give each column's block maximum.
        uint2 xw[EPI == 1 ? PASSES : 1];
        float inv4[4];
        bool nf4[4];
        if (EPI == 1) {
            const int cx = col0 + (lane % LANES_PER_ROW) * CHUNK_ELEMS;
            const bool xvec = (N % 4) == 0 && cx + 4 <= N;
            uint32_t m4[4] = {0u, 0u, 0u, 0u};
#pragma unroll
            for (int p = 0; p < PASSES; ++p) {
                const int row = rbase + p * ROWS_PER_PASS + lane / LANES_PER_ROW;
                uint2 w = make_uint2(0u, 0u);
                if (row < M) {
                    const uint16_t* xr = ex + (int64_t)row * N + cx;
                    if (xvec) {
                        w = *(const uint2*)xr;
                    } else {
                        uint32_t e4[4];
#pragma unroll
                        for (int e = 0; e < 4; ++e) e4[e] = cx + e < N ? (uint32_t)xr[e] : 0u;
                        w = make_uint2(e4[0] | (e4[1] << 16), e4[2] | (e4[3] << 16));
                    }
                }
                xw[p] = w;
                m4[0] = max(m4[0], (w.x << 16) & 0x7FFFFFFFu);
                m4[1] = max(m4[1], w.x & 0x7FFF0000u);
                m4[2] = max(m4[2], (w.y << 16) & 0x7FFFFFFFu);
                m4[3] = max(m4[3], w.y & 0x7FFF0000u);
            }
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                m4[e] = max(m4[e], (uint32_t)__shfl_xor((int)m4[e], 16));
                m4[e] = max(m4[e], (uint32_t)__shfl_xor((int)m4[e], 32));
                nf4[e] = m4[e] >= 0x7F800000u;
                inv4[e] = e8m0_inv_scale_f32(nf4[e] ? 0u : e8m0_from_amax(m4[e]));
            }
        }
#pragma unroll
        for (int p = 0; p < PASSES; ++p) {
            const int rl = p * ROWS_PER_PASS + lane / LANES_PER_ROW;
            const int ce = (lane % LANES_PER_ROW) * CHUNK_ELEMS;
            // 96-column waves: lanes past the last whole row, and rows past 32
            if (lane >= ROWS_PER_PASS * LANES_PER_ROW || rl >= 32) continue;
            u32x4 v = *(const u32x4*)(reg + rl * PITCH + ce * ESZ);
            if (EPI == 1) {
                // the gradient estimator's product, as fp4q_grad_estimate forms it
                const float xf[4] = {bf16_lo(xw[p].x), bf16_hi(xw[p].x), bf16_lo(xw[p].y),
                                     bf16_hi(xw[p].y)};
                float o[4] = {as_f32(v.x), as_f32(v.y), as_f32(v.z), as_f32(v.w)};
#pragma unroll
                for (int e = 0; e < 4; ++e)
                    o[e] = o[e] * (nf4[e] ? __builtin_nanf("") : dge_factor(xf[e], inv4[e], dp));
                v = (u32x4){as_u32(o[0]), as_u32(o[1]), as_u32(o[2]), as_u32(o[3])};
            }
            const int row = rbase + rl;
            const int col = col0 + ce;
            if (row >= M) continue;
            if (EPI == 2) {
                // 8 bf16 of one row; 4 adjacent lanes hold a 32-column block
                // (the ROW quantiser's steps: bit amax, E8M0 byte, scaled
                // nearest-even converts; a non-finite block: 0xFF and zero codes)
                const u16x2_t m0 = __builtin_bit_cast(u16x2_t, v.x & 0x7FFF7FFFu);
                const u16x2_t m1 = __builtin_bit_cast(u16x2_t, v.y & 0x7FFF7FFFu);
                const u16x2_t m2 = __builtin_bit_cast(u16x2_t, v.z & 0x7FFF7FFFu);
                const u16x2_t m3 = __builtin_bit_cast(u16x2_t, v.w & 0x7FFF7FFFu);
                const u16x2_t mm = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1),
                                                             __builtin_elementwise_max(m2, m3));
                const uint32_t amax = group_max_u32<4>(((uint32_t)max(mm.x, mm.y)) << 16);
                const bool nonfinite = amax >= 0x7F800000u;
                const uint32_t byte = nonfinite ? 0xFFu : e8m0_from_amax(amax);
                const float sc = e8m0_scale_f32(byte);
                // the words go through scalars: this compiler, given a
                // bit-cast of a vector element straight into the convert
                // builtin, feeds element 0 to all four converts
                const uint32_t w0 = v.x, w1 = v.y, w2 = v.z, w3 = v.w;
                uint32_t packed = 0;
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w0), sc, 0);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w1), sc, 1);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w2), sc, 2);
                packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(
                    packed, __builtin_bit_cast(bf16x2_t, w3), sc, 3);
                if (nonfinite) packed = 0;
                if (col < N) {
                    *(uint32_t*)(qc + (int64_t)row * (N / 2) + col / 2) = packed;
                    if ((lane & 3) == 0) qs[(int64_t)row * (N / 32) + col / 32] = (uint8_t)byte;
                }
                if (!cptr) continue;
            }
            const int64_t off = (int64_t)row * ldc + col;
            if (vec_ok && col + CHUNK_ELEMS <= N) {
                // C is written once and not read again by this kernel:
                // non-temporal stores keep it from displacing the operands in
                // the caches (worth 10% on a 906 MB fp32 C)
                if (ACCUM) {
                    float4 o = YPF ? yv[YPF ? p : 0] : *(const float4*)((const float*)cptr + off);
                    o.x += as_f32(v.x);
                    o.y += as_f32(v.y);
                    o.z += as_f32(v.z);
                    o.w += as_f32(v.w);
                    __builtin_nontemporal_store(
                        (u32x4){as_u32(o.x), as_u32(o.y), as_u32(o.z), as_u32(o.w)},
                        (u32x4*)((float*)cptr + off));
                } else if (OUT_BF16) {
                    __builtin_nontemporal_store(v, (u32x4*)((uint16_t*)cptr + off));
                } else {
                    __builtin_nontemporal_store(v, (u32x4*)((float*)cptr + off));
                }
            } else {
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < CHUNK_ELEMS; ++e) {
                    if (col + e >= N) break;
                    if (OUT_BF16) {
                        ((uint16_t*)cptr)[off + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                    } else if (ACCUM) {
                        ((float*)cptr)[off + e] += as_f32(w[e]);
                    } else {
                        ((float*)cptr)[off + e] = as_f32(w[e]);
                    }
                }
            }
        }
        __builtin_amdgcn_wave_barrier();
    };
    if constexpr (YPF) {
        c_prefetch(0, ya);
        c_prefetch(1, yb);
        epi_group(0, ya);
        c_prefetch(2, ya);
        epi_group(1, yb);
        c_prefetch(3, yb);
        epi_group(2, ya);
        epi_group(3, yb);
    } else {
#pragma unroll
        for (int i = 0; i < TM; ++i) epi_group(i, ya);
    }
#endif
}

// ---------------------------------------------------------------------------
// Persistent form: one workgroup per compute unit walks tiles blockIdx.x,
// blockIdx.x + gridDim.x, ... and the operand ring runs on across tile
// boundaries: the last three K steps of a tile issue the next tile's first
// three steps (and its first scale group), so those loads are in flight
// while the tile's epilogue stores C, and the next tile starts without a
// relaunch or a cold first load.  For K % 1024 == 0 (the K steps of a tile a
// multiple of 8, so each tile starts at step 0 of the unrolled turn and of a
// scale group; HALF: K % 2048 == 1024, a tile ends on a half turn and its
// first scale buffer alternates from tile to tile) and plain C; the epilogue
// stages each wave's rows in the stage and the scale buffer the tile's last
// step and last group used (st3 and that buffer), which the next tile does
// not touch before the barrier that ends the epilogue.  Every output is
// summed over K in the same order as the one-tile-per-workgroup kernel, so
// the two agree bit for bit.
struct TileRsrc {
    __amdgpu_buffer_rsrc_t ra, rb, rsc;
};

// Origin of tile number t (XCD-contiguous, then grouped along M, as the
// one-tile kernel maps its workgroups).
__device__ __forceinline__ void tile_origin(int t, int ntiles, int tiles_m, int tiles_n, int& m0,
                                            int& n0) {
    using L = Layout<0>;
    int wg = t;
    const int full = (ntiles / 8) * 8;
    if (wg < full) wg = (wg % 8) * (full / 8) + wg / 8;
    const int per_group = GROUP_M * tiles_n;
    const int grp = wg / per_group;
    const int first_m = grp * GROUP_M;
    const int gsize = min(GROUP_M, tiles_m - first_m);
    const int in_grp = wg - grp * per_group;
    m0 = (first_m + in_grp % gsize) * L::BM;
    n0 = (in_grp / gsize) * L::BN;
}

__device__ __forceinline__ TileRsrc tile_rsrc(const uint8_t* ac, const uint8_t* as,
                                              const uint8_t* bc, const uint8_t* bs, int M, int N,
                                              int m0, int n0, int kbytes, int kscale, int wave) {
#if defined(__HIP_DEVICE_COMPILE__)
    using L = Layout<0>;
    const int rows_a = min(M - m0, L::BM), rows_b = min(N - n0, L::BN);
    TileRsrc r;
    r.ra = __builtin_amdgcn_make_buffer_rsrc((void*)(ac + (int64_t)m0 * kbytes), (short)0,
                                             rows_a * kbytes, BUF_FLAGS);
    r.rb = __builtin_amdgcn_make_buffer_rsrc((void*)(bc + (int64_t)n0 * kbytes), (short)0,
                                             rows_b * kbytes, BUF_FLAGS);
    r.rsc = wave < L::A_SWAVES
                ? __builtin_amdgcn_make_buffer_rsrc((void*)(as + (int64_t)m0 * kscale), (short)0,
                                                    rows_a * kscale, BUF_FLAGS)
                : __builtin_amdgcn_make_buffer_rsrc((void*)(bs + (int64_t)n0 * kscale), (short)0,
                                                    rows_b * kscale, BUF_FLAGS);
    return r;
#else
    return TileRsrc{};
#endif
}

// Epilogue of the persistent form: C rows of this wave's tile, staged CW
// columns at a time in `reg` (32 rows x (CW * ESZ + 16) bytes), then written
// as 16-byte chunks with non-temporal stores (or added into an fp32 C).
template <int OUT_BF16, int ACCUM>
__device__ __forceinline__ void persist_epilogue(v16f (&acc)[4][2], uint8_t* reg, void* cptr,
                                                 int64_t ldc, int M, int N, int row0, int col0,
                                                 int lane) {
    using L = Layout<0>;
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int CW = OUT_BF16 ? 64 : 32;  // columns staged per pass
    constexpr int JPC = CW / 32;            // MFMA tiles per pass
    constexpr int PITCH = CW * ESZ + 16;
    constexpr int CHUNK_ELEMS = 16 / ESZ;
    constexpr int LANES_PER_ROW = CW / CHUNK_ELEMS;
    constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;
    constexpr int PASSES = 32 / ROWS_PER_PASS;
    const int half = lane >> 5, l32 = lane & 31;
    const bool vec_ok = ((ldc * ESZ) % 16 == 0) && (((uintptr_t)cptr & 15) == 0);
#pragma unroll
    for (int i = 0; i < L::TM; ++i) {
#pragma unroll
        for (int jc = 0; jc < L::TN / JPC; ++jc) {
#pragma unroll
            for (int jj = 0; jj < JPC; ++jj)
#pragma unroll
                for (int g = 0; g < 4; ++g) {
                    const int j = jc * JPC + jj;
                    const int cl = jj * 32 + 8 * g + 4 * half;
                    uint8_t* dst = reg + l32 * PITCH + cl * ESZ;
                    const v16f& a = acc[i][j];
                    if (OUT_BF16) {
                        const bf16x2_t p0 = {(__bf16)a[4 * g], (__bf16)a[4 * g + 1]};
                        const bf16x2_t p1 = {(__bf16)a[4 * g + 2], (__bf16)a[4 * g + 3]};
                        *(uint2*)dst = make_uint2(__builtin_bit_cast(uint32_t, p0),
                                                  __builtin_bit_cast(uint32_t, p1));
                    } else {
                        *(u32x4*)dst = (u32x4){as_u32(a[4 * g]), as_u32(a[4 * g + 1]),
                                               as_u32(a[4 * g + 2]), as_u32(a[4 * g + 3])};
                    }
                }
            __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0)
            __builtin_amdgcn_wave_barrier();
#pragma unroll
            for (int p = 0; p < PASSES; ++p) {
                const int rl = p * ROWS_PER_PASS + lane / LANES_PER_ROW;
                const int ce = (lane % LANES_PER_ROW) * CHUNK_ELEMS;
                const u32x4 v = *(const u32x4*)(reg + rl * PITCH + ce * ESZ);
                const int row = row0 + i * 32 + rl;
                const int col = col0 + jc * CW + ce;
                if (row >= M) continue;
                const int64_t off = (int64_t)row * ldc + col;
                if (vec_ok && col + CHUNK_ELEMS <= N) {
                    if (ACCUM) {
                        float4 o = __builtin_bit_cast(
                            float4,
                            __builtin_nontemporal_load((const u32x4*)((const float*)cptr + off)));
                        o.x += as_f32(v.x);
                        o.y += as_f32(v.y);
                        o.z += as_f32(v.z);
                        o.w += as_f32(v.w);
                        __builtin_nontemporal_store(
                            (u32x4){as_u32(o.x), as_u32(o.y), as_u32(o.z), as_u32(o.w)},
                            (u32x4*)((float*)cptr + off));
                    } else if (OUT_BF16) {
                        __builtin_nontemporal_store(v, (u32x4*)((uint16_t*)cptr + off));
                    } else {
                        __builtin_nontemporal_store(v, (u32x4*)((float*)cptr + off));
                    }
                } else {
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < CHUNK_ELEMS; ++e) {
                        if (col + e >= N) break;
                        if (OUT_BF16) {
                            ((uint16_t*)cptr)[off + e] = (uint16_t)(w[e >> 1] >> (16 * (e & 1)));
                        } else if (ACCUM) {
                            ((float*)cptr)[off + e] += as_f32(w[e]);
                        } else {
                            ((float*)cptr)[off + e] = as_f32(w[e]);
                        }
                    }
                }
            }
            __builtin_amdgcn_wave_barrier();
        }
    }
}

template <int OUT_BF16, int ACCUM, int HALF>
__global__ __launch_bounds__(Layout<0>::THREADS, 1) void gemm_fp4_persistent_kernel(
    int M, int N, int K, const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, void* __restrict__ cptr,
    int64_t ldc, int tiles_m, int tiles_n) {
#if defined(__HIP_DEVICE_COMPILE__)
    using L = Layout<0>;
    constexpr int CFG = 0, BF16OPS = 0, TAIL = 0, SG = 8;
    constexpr int TM = L::TM, TN = L::TN;
    const int ntiles = tiles_m * tiles_n;
    const int G = gridDim.x;
    int tseq = blockIdx.x;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / L::WN, wn = wave % L::WN;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    const int off0 = (l32 >> 4) * REGION + region_slot(l32 & 15, half) * 16;
    const int off1 = (l32 >> 4) * REGION + region_slot(l32 & 15, 2 + half) * 16;
    const int sxor = (l32 >> 3) & 3;
    const int kbytes = K / 2;
    const int kscale = K / 32;
    const int ksteps = kbytes / BKB;  // a multiple of 16, or of 8 with HALF

    // Workgroups that own one tile fewer than the others (those past
    // ntiles % G in the deal) have a whole tile of slack.  They start about a
    // fifth of a tile late (0.2 us per K step, in 10 ns ticks of the real-time
    // counter; a K step takes about 1 us), so that the workgroups on the
    // critical path issue their first loads, and later write their first
    // tiles, without them: 8192 x 5632 x 2048 60.1 -> 57.2 us, 4096 x 5632 x
    // 2048 36.7 -> 35.0 us on one MI355X.  A bounded wait on a clock, no
    // dependence on other workgroups.
    {
        const int most = (ntiles + G - 1) / G;
        const int mine = (ntiles - (int)blockIdx.x + G - 1) / G;
        if (mine < most) {
            constexpr uint64_t kTicksPerStep = 20;
            const uint64_t until =
                __builtin_amdgcn_s_memrealtime() + (uint64_t)ksteps * kTicksPerStep;
            while (__builtin_amdgcn_s_memrealtime() < until) __builtin_amdgcn_s_sleep(16);
        }
    }

    // per-lane offsets, the same for every tile
    Src<CFG> src;
    {
        const int j = lane >> 2;
        const int c = (lane & 3) ^ ((j >> 2) & 3);
#pragma unroll
        for (int q = 0; q < L::RPW; ++q)
            src.vrow[q] = (uint32_t)(((q * L::WAVES + wave) * 16 + j) * kbytes + c * 16);
        constexpr int HW = L::A_SWAVES;
        const int sbase = ((wave < HW ? wave : wave - HW) * L::SROWS + (lane >> 3)) * kscale;
#pragma unroll
        for (int q = 0; q < 4; ++q) src.vsc[q] = (uint32_t)(sbase + (((lane & 7) ^ q) << 2));
        src.soff = 0;
    }
    int m0, n0, m1 = 0, n1 = 0;
    tile_origin(tseq, ntiles, tiles_m, tiles_n, m0, n0);
    TileRsrc cur = tile_rsrc(ac, as, bc, bs, M, N, m0, n0, kbytes, kscale, wave), nxt = cur;
    bool has_next = tseq + G < ntiles;
    if (has_next) {
        tile_origin(tseq + G, ntiles, tiles_m, tiles_n, m1, n1);
        nxt = tile_rsrc(ac, as, bc, bs, M, N, m1, n1, kbytes, kscale, wave);
    }

    Frags<CFG> FA, FB;
    uint32_t sa[TM], ra[TM], sb[TN], rb[TN];
#pragma unroll
    for (int i = 0; i < TM; ++i) sa[i] = ra[i] = 0;
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[j] = rb[j] = 0;
    const int sh = 8 * half;
    constexpr int LC = L::RPW_A + L::RPW_B;

    // first tile: scale group 0 and code steps 0..2
    src.ra = cur.ra;
    src.rb = cur.rb;
    src.rsc = cur.rsc;
    issue_scale_pieces<CFG, 0, L::SPIECES, 0>(src, sc0, wave, kscale, 0);
    src.soff = 0;
    issue_codes<CFG, 0>(src, st0, wave, true);
    issue_codes<CFG, 0>(src, st1, wave, true);
    issue_codes<CFG, 0>(src, st2, wave, true);
    FP4Q_WAIT_VMCNT(2 * LC);
    __builtin_amdgcn_s_barrier();
    read_scales<CFG, 0>(sc0, sxor << 2, wm, wn, lane, ra, rb);
    read_frags<CFG>(st0, off0, wm, wn, FA);

#define FP4Q_PIECES(p) ((((p) & 7) >= 4) ? 0 : L::SPIECES / 4)
#define FP4Q_BEHIND(p) (FP4Q_PIECES((p) + 6) + LC + FP4Q_PIECES((p) + 7) + LC + FP4Q_PIECES(p))
    // Scale group j of a tile uses buffer (j + ph_) % 2, ph_ being the buffer
    // of the tile's first group: 0 for every tile when a tile has an even
    // number of 8-step groups; with HALF (K % 2048 == 1024: 16-step turns and
    // a last half turn, an odd number of groups) it alternates from tile to
    // tile, and each parity has its own copy of the tile's code, so that
    // every LDS buffer is still named at compile time.
#define FP4Q_SCUR(P) (((((P) / SG) + ph_) & 1) ? sc1 : sc0)
#define FP4Q_SNXT(P) (((((P) / SG) + ph_) & 1) ? sc0 : sc1)
    // one K step; the loads it issues (step t_ + 3 and, early in a scale
    // group, the next group's pieces) come from this tile or, past its end,
    // from the next one (or repeat this tile's last step when there is none)
#define FP4Q_PSTEP(P, CUR, NEXT1, NEXTL)                                             \
    do {                                                                             \
        const int t_ = kt + (P);                                                     \
        __builtin_amdgcn_sched_barrier(0);                                           \
        shift_scales<CFG>(ra, rb, sh, sa, sb);                                       \
        read_frags<CFG>(CUR, off1, wm, wn, FB);                                       \
        {                                                                            \
            const int tl_ = t_ + 3;                                                  \
            const bool into_next_ = tl_ >= ksteps && has_next;                       \
            const TileRsrc& r_ = into_next_ ? nxt : cur;                             \
            src.ra = r_.ra;                                                          \
            src.rb = r_.rb;                                                          \
            src.soff = (into_next_ ? tl_ - ksteps : min(tl_, ksteps - 1)) * BKB;     \
            issue_codes<CFG, 0>(src, NEXTL, wave, false);                            \
        }                                                                            \
        if (FP4Q_PIECES(P)) {                                                        \
            const int g_ = t_ / SG + 1;                                              \
            const bool into_next_ = g_ * SG >= ksteps && has_next;                   \
            src.rsc = into_next_ ? nxt.rsc : cur.rsc;                                \
            issue_scale_pieces<CFG, ((P) & 3) * (L::SPIECES / 4), L::SPIECES / 4, 0>(     \
                src, FP4Q_SNXT(P), wave, kscale, into_next_ ? 0 : g_);               \
        }                                                                            \
        __builtin_amdgcn_sched_barrier(0);                                           \
        mfma_half<CFG, 0, 0>(FA, sa, sb, acc);                                       \
        __builtin_amdgcn_sched_barrier(0);                                           \
        FP4Q_WAIT_VMCNT(FP4Q_BEHIND(P));                                             \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                          \
        __builtin_amdgcn_s_barrier();                                                \
        __builtin_amdgcn_sched_barrier(0);                                           \
        read_scales<CFG, 0>(((P) % SG) == SG - 1 ? FP4Q_SNXT(P) : FP4Q_SCUR(P),      \
                            (((P) + 1) & 7 ^ sxor) << 2, wm, wn, lane, ra, rb);      \
        read_frags<CFG>(NEXT1, off0, wm, wn, FA);                                     \
        mfma_half<CFG, 0, 1>(FB, sa, sb, acc);                                       \
    } while (0)

    // One tile: its K steps (turns of 16; with HALF the last turn stops after
    // its first 8 steps),
    // its epilogue through the stage and the scale buffer that its last step
    // and last group used (six waves' regions in st3, two in SC_LAST), then
    // on to the next tile, whose first scale group sits in SC_FIRST.  The
    // scale group j of a tile uses buffer (j + PH) % 2; with HALF (an odd
    // number of groups per tile) PH alternates, so the loop body holds two
    // tiles, one of each parity, and every LDS buffer is still named at
    // compile time.
#define FP4Q_TILE(PH, SC_LAST, SC_FIRST)                                                \
    {                                                                                   \
        constexpr int ph_ = (PH);                                                       \
        v16f acc[TM][TN];                                                               \
        _Pragma("unroll") for (int i = 0; i < TM; ++i)                                  \
        _Pragma("unroll") for (int j = 0; j < TN; ++j)                                  \
        _Pragma("unroll") for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;             \
        for (int kt = 0; kt < ksteps; kt += 16) {                                       \
            FP4Q_PSTEP(0, st0, st1, st3);                                           \
            FP4Q_PSTEP(1, st1, st2, st0);                                           \
            FP4Q_PSTEP(2, st2, st3, st1);                                           \
            FP4Q_PSTEP(3, st3, st0, st2);                                           \
            FP4Q_PSTEP(4, st0, st1, st3);                                           \
            FP4Q_PSTEP(5, st1, st2, st0);                                           \
            FP4Q_PSTEP(6, st2, st3, st1);                                           \
            FP4Q_PSTEP(7, st3, st0, st2);                                           \
            if (!HALF || kt + 16 <= ksteps) {                                           \
                FP4Q_PSTEP(8, st0, st1, st3);                                       \
                FP4Q_PSTEP(9, st1, st2, st0);                                       \
                FP4Q_PSTEP(10, st2, st3, st1);                                      \
                FP4Q_PSTEP(11, st3, st0, st2);                                      \
                FP4Q_PSTEP(12, st0, st1, st3);                                      \
                FP4Q_PSTEP(13, st1, st2, st0);                                      \
                FP4Q_PSTEP(14, st2, st3, st1);                                      \
                FP4Q_PSTEP(15, st3, st0, st2);                                      \
            }                                                                           \
        }                                                                               \
        {                                                                               \
            constexpr int ESZ = OUT_BF16 ? 2 : 4;                                       \
            constexpr int CW = OUT_BF16 ? 64 : 32;                                      \
            constexpr int EREG = 32 * (CW * ESZ + 16);                                  \
            static_assert(6 * EREG <= STAGE && 2 * EREG <= SCALE_BUF, "staging fits");  \
            uint8_t* reg = wave < 6 ? st3 + wave * EREG : (SC_LAST) + (wave - 6) * EREG; \
            persist_epilogue<OUT_BF16, ACCUM>(acc, reg, cptr, ldc, M, N,                \
                                              m0 + wm * L::WROWS, n0 + wn * L::WCOLS, lane); \
        }                                                                               \
        __syncthreads(); /* the staging buffers are free before the next tile refills them */ \
        if (!has_next) break;                                                           \
        tseq += G;                                                                      \
        m0 = m1;                                                                        \
        n0 = n1;                                                                        \
        cur = nxt;                                                                      \
        has_next = tseq + G < ntiles;                                                   \
        if (has_next) {                                                                 \
            tile_origin(tseq + G, ntiles, tiles_m, tiles_n, m1, n1);                    \
            nxt = tile_rsrc(ac, as, bc, bs, M, N, m1, n1, kbytes, kscale, wave);        \
        }                                                                               \
        /* the next tile's step 0 and scale group 0 landed before the last step's */    \
        /* barrier; read them again (nothing was kept across the epilogue) */           \
        read_scales<CFG, 0>(SC_FIRST, sxor << 2, wm, wn, lane, ra, rb);                 \
        read_frags<CFG>(st0, off0, wm, wn, FA);                                          \
    }
    for (;;) {
        if (HALF) {
            FP4Q_TILE(0, sc0, sc1)
            FP4Q_TILE(1, sc1, sc0)
        } else {
            FP4Q_TILE(0, sc1, sc0)
        }
    }
#undef FP4Q_TILE
#undef FP4Q_PSTEP
#undef FP4Q_PIECES
#undef FP4Q_BEHIND
#undef FP4Q_SCUR
#undef FP4Q_SNXT
    FP4Q_WAIT_VMCNT(0);  // the repeated loads of the last step have landed
    (void)TAIL;
    (void)BF16OPS;
#endif
}

// Compute units of the current device (cached per device).
static int device_cus() {
    static int cache[64] = {0};
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    if (cache[dev] == 0) {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
            n <= 0)
            n = 256;
        cache[dev] = n;
    }
    return cache[dev];
}

// Tile configuration for an M x N output: one workgroup per compute unit at
// a time, so the time goes as (rounds of workgroups) x (time per tile).  A
// 128 x 384 tile holds 3/4 of a 256 x 256 tile's work but, measured on
// MI355X, takes about 1.09x its time (its half-step of 6 MFMAs per wave hides
// less of the LDS latency, and it loads 4/3 the operand bytes per flop), so
// it is taken only where it saves a whole round (e.g. 257 tiles of 256 x 256
// against at most 256 of 128 x 384).
// FP4Q_GEMM_TILE=256x256 or 128x384 in the environment forces one (tests
// cover both on the same shapes).
static int pick_cfg(int64_t M, int64_t N) {
    if (const char* e = getenv("FP4Q_GEMM_TILE")) {
        if (!strcmp(e, "256x256")) return 0;
        if (!strcmp(e, "128x384")) return 1;

    }
    const int64_t cus = device_cus();
    const int64_t t0 = ((M + 255) / 256) * ((N + 255) / 256);
    const int64_t t1 = ((M + 127) / 128) * ((N + 383) / 384);
    const double e0 = (double)((t0 + cus - 1) / cus);
    const double e1 = (double)((t1 + cus - 1) / cus) * 1.09;
    return e1 < e0 ? 1 : 0;
}

template <int CFG, int OUT_BF16, int ACCUM, int OPS, int EPI = 0>
static void launch_cfg(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                       const uint8_t* b, const uint8_t* bs, void* c, int64_t ldc, hipStream_t s,
                       const uint8_t* ha, const uint8_t* hb, int64_t kp,
                       const uint16_t* ex = nullptr, DgeParams dp = DgeParams{},
                       uint8_t* qc = nullptr, uint8_t* qs = nullptr) {
    using L = Layout<CFG>;
    const int tiles_m = (int)((M + L::BM - 1) / L::BM);
    const int tiles_n = (int)((N + L::BN - 1) / L::BN);
    const dim3 grid((unsigned)(tiles_m * tiles_n));
    // an FP4 K loop that ends on a half step (K % 128 == 64) takes the TAIL form
    if constexpr (OPS != 1) {
        if (K % 128) {
            FP4Q_LAUNCH((gemm_fp4_kernel<CFG, OUT_BF16, ACCUM, OPS, EPI, 1>), grid,
                        dim3(L::THREADS), 0, s, (int)M, (int)N, (int)K, a, as, b, bs, c, ldc,
                        tiles_m, tiles_n, ha, hb, (int)kp, ex, dp, qc, qs);
            return;
        }
    }
    // the accumulating bf16 form takes the first round's size in kp (see the kernel)
    if constexpr (OPS == 1 && ACCUM) {
        const int64_t cus = device_cus();
        kp = (int64_t)tiles_m * tiles_n > 2 * cus ? cus : 0;
    }
    FP4Q_LAUNCH((gemm_fp4_kernel<CFG, OUT_BF16, ACCUM, OPS, EPI, 0>), grid, dim3(L::THREADS), 0, s,
                (int)M, (int)N, (int)K, a, as, b, bs, c, ldc, tiles_m, tiles_n, ha, hb, (int)kp,
                ex, dp, qc, qs);
}

// Whether the persistent form runs: plain FP4 GEMMs on 256 x 256 tiles with
// K % 1024 == 0 and more tiles than compute units (FP4Q_GEMM_PERSIST=0
// disables it, =1 forces it wherever it applies).
static bool use_persistent(int64_t M, int64_t N, int64_t K) {
    if (K % 1024) return false;
    const char* e = getenv("FP4Q_GEMM_PERSIST");
    if (e && !strcmp(e, "0")) return false;
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    if (e && !strcmp(e, "1")) return true;
    return tiles > device_cus();
}

template <int OUT_BF16, int ACCUM, int OPS>
static void launch_tiles(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                         const uint8_t* b, const uint8_t* bs, void* c, int64_t ldc,
                         hipStream_t s, const uint8_t* ha = nullptr, const uint8_t* hb = nullptr,
                         int64_t kp = 0) {
    if constexpr (OPS == 0) {
        if (pick_cfg(M, N) == 0 && use_persistent(M, N, K)) {
            const int tiles_m = (int)((M + 255) / 256), tiles_n = (int)((N + 255) / 256);
            const int ntiles = tiles_m * tiles_n;
            int64_t grid = std::min<int64_t>(ntiles, device_cus());
            // FP4Q_GEMM_PERSIST_GRID=g caps the number of workgroups (so that
            // tests can chain several tiles per workgroup at small sizes)
            if (const char* g = getenv("FP4Q_GEMM_PERSIST_GRID")) {
                const long v = strtol(g, nullptr, 10);
                if (v > 0) grid = std::min<int64_t>(grid, v);
            }
            if (K % 2048)
                FP4Q_LAUNCH((gemm_fp4_persistent_kernel<OUT_BF16, ACCUM, 1>),
                            dim3((unsigned)grid), dim3(512), 0, s, (int)M, (int)N, (int)K, a, as,
                            b, bs, c, ldc, tiles_m, tiles_n);
            else
                FP4Q_LAUNCH((gemm_fp4_persistent_kernel<OUT_BF16, ACCUM, 0>),
                            dim3((unsigned)grid), dim3(512), 0, s, (int)M, (int)N, (int)K, a, as,
                            b, bs, c, ldc, tiles_m, tiles_n);
            return;
        }
    }
    if (pick_cfg(M, N) == 1)
        launch_cfg<1, OUT_BF16, ACCUM, OPS>(M, N, K, a, as, b, bs, c, ldc, s, ha, hb, kp);
    else
        launch_cfg<0, OUT_BF16, ACCUM, OPS>(M, N, K, a, as, b, bs, c, ldc, s, ha, hb, kp);
}

hipError_t launch_gemm_fp4(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                           const uint8_t* as, const uint8_t* bc, const uint8_t* bs, void* c,
                           int cdtype, int64_t ldc, bool accumulate, hipStream_t s) {
    if (cdtype == BF16)
        launch_tiles<1, 0, 0>(M, N, K, ac, as, bc, bs, c, ldc, s);
    else if (accumulate)
        launch_tiles<0, 1, 0>(M, N, K, ac, as, bc, bs, c, ldc, s);
    else
        launch_tiles<0, 0, 0>(M, N, K, ac, as, bc, bs, c, ldc, s);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16_accum(int64_t M, int64_t N, int64_t K, const uint16_t* a,
                                  const uint16_t* b, float* c, int64_t ldc, hipStream_t s) {
    launch_tiles<0, 1, 1>(M, N, K, (const uint8_t*)a, nullptr, (const uint8_t*)b, nullptr, c, ldc,
                          s);
    return hipGetLastError();
}

hipError_t launch_gemm_fp4_hot(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                               const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                               const uint16_t* ha, const uint16_t* hb, int64_t kp, float* c,
                               int64_t ldc, hipStream_t s) {
    launch_tiles<0, 0, 2>(M, N, K, ac, as, bc, bs, c, ldc, s, (const uint8_t*)ha,
                          (const uint8_t*)hb, kp);
    return hipGetLastError();
}

hipError_t launch_gemm_fp4_dge(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                               const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                               const uint16_t* x, float k, float clamp_max, float* c,
                               int64_t ldc, hipStream_t s) {
    DgeParams P;
    P.invk = 1.0f / k;
    P.p = 1.0f / k - 1.0f;
    P.clamp_max = clamp_max;
    P.k_one = (k == 1.0f);
    launch_cfg<0, 0, 0, 0, 1>(M, N, K, ac, as, bc, bs, c, ldc, s, nullptr, nullptr, 0, x, P);
    return hipGetLastError();
}

hipError_t launch_gemm_fp4_quant(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                                 const uint8_t* as, const uint8_t* bc, const uint8_t* bs,
                                 uint16_t* c, int64_t ldc, uint8_t* qc, uint8_t* qs,
                                 hipStream_t s) {
    launch_cfg<0, 1, 0, 0, 2>(M, N, K, ac, as, bc, bs, c, ldc, s, nullptr, nullptr, 0, nullptr,
                              DgeParams{}, qc, qs);
    return hipGetLastError();
}

}  // namespace fp4q
