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
// Tiling: a 256-thread workgroup (4 waves, 2 x 2) computes a 256 x 256 tile
// of C; each wave a 128 x 128 sub-tile as 4 x 4 MFMA tiles (256 accumulator
// registers).  The K loop steps 128 elements (64 bytes per row): A and B
// tiles go global -> registers -> LDS in MFMA fragment order (fragment =
// 32 rows x 32 bytes, lane l's 16 bytes at l*16), so every LDS read and
// write is a conflict-free 16-byte-per-lane access; LDS is double-buffered
// and the next K step's global loads are in flight while the current one
// runs on the MFMA units.  Scale words (4 bytes per row per K step) are
// loaded straight into registers one step ahead.  Workgroups are remapped
// so that consecutive tiles of a grouped (4 tile-rows) order run on the same
// XCD and share its L2.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __attribute__((address_space(3))) void* lds_ptr_t;
// Native 4 x 32-bit vectors (HIP's uint4 is a class with unions, which the
// compiler does not always split into registers).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

static constexpr int BM = 256, BN = 256;
static constexpr int BKB = 64;  // K bytes per step (128 fp4 elements)
static constexpr int kThreads = 256;
static constexpr int FRAG = 1024;               // bytes per LDS fragment
#ifndef FP4Q_GEMM_NSTAGE
#define FP4Q_GEMM_NSTAGE 3
#endif
static constexpr int NSTAGE = FP4Q_GEMM_NSTAGE; // LDS ring depth (3 or 4)
static constexpr int OFF_B = 16 * FRAG;         // B fragments within a stage
static constexpr int OFF_SA = 32 * FRAG;        // A scale words (256 x 4 B)
static constexpr int OFF_SB = 32 * FRAG + 1024; // B scale words
static constexpr int STAGE = 32 * FRAG + 2048;
// per wave and K step: 8 fragment loads, plus 2 scale-row loads for FP4
template <int BF16OPS>
struct StepLoads {
    static constexpr int n = BF16OPS ? 8 : 10;
};
static constexpr int GROUP_M = 4;

// s_waitcnt with only the vector-memory counter constrained (gfx9 encoding:
// vmcnt in bits 3:0 and 15:14, expcnt 6:4 and lgkmcnt 11:8 left at maximum).
#define FP4Q_WAIT_VMCNT(n) __builtin_amdgcn_s_waitcnt(((n) & 0xF) | (((n) >> 4) << 14) | 0x0F70)

struct StepSrc {
    const uint8_t* ga[4];
    const uint8_t* gb[4];
    const uint8_t* gsa;
    const uint8_t* gsb;
};

#ifndef FP4Q_GEMM_DMA
#define FP4Q_GEMM_DMA 0
#endif

// Register staging of one K step's operands (used when the loads go
// global -> VGPR -> LDS instead of straight into LDS).
struct StepRegs {
    u32x4 a[4], b[4];
    uint32_t sa, sb;
};

template <int BF16OPS>
__device__ __forceinline__ void load_step(const StepSrc& src, int kt, StepRegs& R) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        R.a[q] = *(const u32x4*)(src.ga[q] + (int64_t)kt * BKB);
        R.b[q] = *(const u32x4*)(src.gb[q] + (int64_t)kt * BKB);
    }
    if (!BF16OPS) {
        R.sa = *(const uint32_t*)(src.gsa + kt * 4);
        R.sb = *(const uint32_t*)(src.gsb + kt * 4);
    }
}

template <int BF16OPS>
__device__ __forceinline__ void store_step(const StepRegs& R, uint8_t* stage, int wave, int lane) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int f = wave * 4 + q;
        *(u32x4*)(stage + f * FRAG + lane * 16) = R.a[q];
        *(u32x4*)(stage + OFF_B + f * FRAG + lane * 16) = R.b[q];
    }
    if (!BF16OPS) {
        *(uint32_t*)(stage + OFF_SA + wave * 256 + lane * 4) = R.sa;
        *(uint32_t*)(stage + OFF_SB + wave * 256 + lane * 4) = R.sb;
    }
}

// Issue the direct-to-LDS loads of K step kt of this wave into `stage`.
template <int BF16OPS>
__device__ __forceinline__ void issue_step(const StepSrc& src, int kt, uint8_t* stage, int wave) {
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int f = wave * 4 + q;
        __builtin_amdgcn_global_load_lds((const void*)(src.ga[q] + (int64_t)kt * BKB),
                                         (lds_ptr_t)(stage + f * FRAG), 16, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(src.gb[q] + (int64_t)kt * BKB),
                                         (lds_ptr_t)(stage + OFF_B + f * FRAG), 16, 0, 0);
    }
    if (!BF16OPS) {
        __builtin_amdgcn_global_load_lds((const void*)(src.gsa + kt * 4),
                                         (lds_ptr_t)(stage + OFF_SA + wave * 256), 4, 0, 0);
        __builtin_amdgcn_global_load_lds((const void*)(src.gsb + kt * 4),
                                         (lds_ptr_t)(stage + OFF_SB + wave * 256), 4, 0, 0);
    }
}

struct Frags {
    u32x4 a[4], b[4];
};

// This wave's A and B fragments of half kk (K bytes kk*32 .. kk*32+31) of a
// staged step: 8 conflict-free 16-byte LDS reads.
__device__ __forceinline__ void read_frags(const uint8_t* base, int kk, int wm, int wn, int lane,
                                           Frags& F) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        F.a[i] = *(const u32x4*)(base + ((wm * 4 + i) * 2 + kk) * FRAG + lane * 16);
        F.b[i] = *(const u32x4*)(base + OFF_B + ((wn * 4 + i) * 2 + kk) * FRAG + lane * 16);
    }
}

// Scale words of this lane's MFMA rows (A) and columns (B), shifted so that
// byte 0 / byte 2 are the K blocks of halves 0 / 1 for this lane's 32-element
// K chunk.
__device__ __forceinline__ void read_scales(const uint8_t* base, int wm, int wn, int lane,
                                            uint32_t (&sa)[4], uint32_t (&sb)[4]) {
    const int half = lane >> 5, l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        sa[i] = *(const uint32_t*)(base + OFF_SA + (wm * 128 + i * 32 + l32) * 4) >> (8 * half);
        sb[i] = *(const uint32_t*)(base + OFF_SB + (wn * 128 + i * 32 + l32) * 4) >> (8 * half);
    }
}

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));

// 16 MFMAs: the 4 x 4 tiles of this wave on half kk of a K step.  FP4: the
// scaled MFMA on E2M1 operands (64 K elements per half); BF16: plain bf16
// MFMAs (16 K elements per half, the same 16 bytes per lane).
template <int BF16OPS>
__device__ __forceinline__ void mfma_half(const Frags& F, const uint32_t (&sa)[4],
                                          const uint32_t (&sb)[4], int kk, v16f (&acc)[4][4]) {
    if (BF16OPS) {
        bf16x8_t ha[4], hb[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            ha[i] = __builtin_bit_cast(bf16x8_t, F.a[i]);
            hb[i] = __builtin_bit_cast(bf16x8_t, F.b[i]);
        }
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(ha[i], hb[j], acc[i][j], 0, 0, 0);
        return;
    }
    v8i fa[4], fb[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        fa[i] = (v8i){(int)F.a[i].x, (int)F.a[i].y, (int)F.a[i].z, (int)F.a[i].w, 0, 0, 0, 0};
        fb[i] = (v8i){(int)F.b[i].x, (int)F.b[i].y, (int)F.b[i].z, (int)F.b[i].w, 0, 0, 0, 0};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fa[i], fb[j], acc[i][j], 4, 4, 0, (int)(sa[i] >> (16 * kk)), 0,
                (int)(sb[j] >> (16 * kk)));
}

template <int OUT_BF16, int ACCUM, int BF16OPS>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp4_kernel(
    int M, int N, int K, const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, void* __restrict__ cptr,
    int64_t ldc, int tiles_m, int tiles_n) {
    // The LDS ring stages are separate objects, so the compiler can tell the
    // stage being read from the stages the in-flight loads write.
    __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[STAGE];
#if FP4Q_GEMM_NSTAGE == 4
    __shared__ __attribute__((aligned(16))) uint8_t st3[STAGE];
#endif

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
    const int m0 = tm * BM, n0 = tn * BN;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    // bytes per operand row; each K step consumes 64 of them
    const int64_t kbytes = BF16OPS ? (int64_t)K * 2 : K / 2;
    const int kscale = K / 32;
    const int ksteps = (int)(kbytes / BKB);
    constexpr int LOADS_PER_STEP = StepLoads<BF16OPS>::n;

    // Global sources of this lane's loads.  Fragment f = rg*2 + kk holds rows
    // rg*32 .. rg*32+31 and K bytes kk*32 .. kk*32+31 of the step; wave w
    // loads fragments 4w .. 4w+3 of A and of B (one 16-byte load per lane,
    // written by the load straight into LDS at fragment base + lane*16), and
    // the scale words of rows 64w .. 64w+63 of A and of B.
    StepSrc src;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int f = wave * 4 + q;
        const int rg = f >> 1, kk = f & 1;
        const int ra = min(m0 + rg * 32 + l32, M - 1);
        const int rb = min(n0 + rg * 32 + l32, N - 1);
        src.ga[q] = ac + (int64_t)ra * kbytes + kk * 32 + half * 16;
        src.gb[q] = bc + (int64_t)rb * kbytes + kk * 32 + half * 16;
    }
    src.gsa = BF16OPS ? nullptr : as + (int64_t)min(m0 + wave * 64 + lane, M - 1) * kscale;
    src.gsb = BF16OPS ? nullptr : bs + (int64_t)min(n0 + wave * 64 + lane, N - 1) * kscale;

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    // Software pipeline over K steps t (LDS ring of NSTAGE stages, two
    // halves kk per step): while the MFMAs of (t, 0) run, the fragments of
    // (t, 1) are read and the loads of step t+NSTAGE-1 are issued; one
    // barrier per step, after which the scales and (t+1, 0) fragments are
    // read while the MFMAs of (t, 1) run.  The barrier follows an lgkmcnt(0)
    // wait, so every wave has finished reading stage t before anyone refills
    // it (at step t+1).
#if FP4Q_GEMM_DMA
#pragma unroll
    for (int s = 0; s < NSTAGE - 1; ++s) {
        uint8_t* stg = s == 0 ? st0 : s == 1 ? st1 : st2;
        if (s < ksteps) issue_step<BF16OPS>(src, s, stg, wave);
    }
    if (ksteps >= NSTAGE - 1) {
        FP4Q_WAIT_VMCNT(LOADS_PER_STEP * (NSTAGE - 2));
    } else {
        FP4Q_WAIT_VMCNT(0);
    }
    __builtin_amdgcn_s_barrier();
    Frags FA, FB;
    uint32_t sa[4] = {0, 0, 0, 0}, sb[4] = {0, 0, 0, 0}, sa_n[4] = {0, 0, 0, 0},
             sb_n[4] = {0, 0, 0, 0};
    if (!BF16OPS) read_scales(st0, wm, wn, lane, sa, sb);
    read_frags(st0, 0, wm, wn, lane, FA);

// One K step.  ISSUE: whether step t+NSTAGE-1 exists (its loads are issued
// here); LAST: whether t is the final step.  Both are compile-time in the
// steady-state loop, so its body has no branches; the few tail steps use
// the run-time form.  sched_barrier(0) keeps the first MFMA half above the
// barrier, so the MFMA pipe has work queued while the wave waits there.
#define FP4Q_GEMM_STEP(t, CUR, NEXT1, NEXTL, ISSUE, LAST)                          \
    do {                                                                           \
        read_frags(CUR, 1, wm, wn, lane, FB);                                      \
        if (ISSUE) issue_step<BF16OPS>(src, (t) + NSTAGE - 1, NEXTL, wave);         \
        mfma_half<BF16OPS>(FA, sa, sb, 0, acc);                                    \
        __builtin_amdgcn_sched_barrier(0);                                         \
        if (ISSUE) {                                                               \
            __builtin_amdgcn_s_waitcnt(((LOADS_PER_STEP * (NSTAGE - 2)) & 0xF) |     \
                                       (((LOADS_PER_STEP * (NSTAGE - 2)) >> 4) << 14) | 0x70); \
        } else {                                                                   \
            __builtin_amdgcn_s_waitcnt(0x70);                                      \
        }                                                                          \
        __builtin_amdgcn_s_barrier();                                              \
        __builtin_amdgcn_sched_barrier(0);                                         \
        if (!(LAST)) {                                                             \
            if (!BF16OPS) read_scales(NEXT1, wm, wn, lane, sa_n, sb_n);            \
            read_frags(NEXT1, 0, wm, wn, lane, FA);                                \
        }                                                                          \
        mfma_half<BF16OPS>(FB, sa, sb, 1, acc);                                    \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) {                            \
            sa[q] = sa_n[q];                                                       \
            sb[q] = sb_n[q];                                                       \
        }                                                                          \
    } while (0)

    // steady state: every step of an unrolled group issues a later step
    int kt = 0;
#if FP4Q_GEMM_NSTAGE == 4
    for (; kt + 3 + NSTAGE - 1 < ksteps; kt += 4) {
        FP4Q_GEMM_STEP(kt, st0, st1, st3, true, false);
        FP4Q_GEMM_STEP(kt + 1, st1, st2, st0, true, false);
        FP4Q_GEMM_STEP(kt + 2, st2, st3, st1, true, false);
        FP4Q_GEMM_STEP(kt + 3, st3, st0, st2, true, false);
    }
    // tail (kt % 4 == 0 here)
    for (; kt < ksteps; kt += 4) {
        FP4Q_GEMM_STEP(kt, st0, st1, st3, kt + NSTAGE - 1 < ksteps, kt + 1 == ksteps);
        if (kt + 1 < ksteps)
            FP4Q_GEMM_STEP(kt + 1, st1, st2, st0, kt + NSTAGE < ksteps, kt + 2 == ksteps);
        if (kt + 2 < ksteps)
            FP4Q_GEMM_STEP(kt + 2, st2, st3, st1, kt + NSTAGE + 1 < ksteps, kt + 3 == ksteps);
        if (kt + 3 < ksteps)
            FP4Q_GEMM_STEP(kt + 3, st3, st0, st2, kt + NSTAGE + 2 < ksteps, kt + 4 == ksteps);
    }
#else
    for (; kt + 2 + NSTAGE - 1 < ksteps; kt += 3) {
        FP4Q_GEMM_STEP(kt, st0, st1, st2, true, false);
        FP4Q_GEMM_STEP(kt + 1, st1, st2, st0, true, false);
        FP4Q_GEMM_STEP(kt + 2, st2, st0, st1, true, false);
    }
    // tail (kt % 3 == 0 here)
    for (; kt < ksteps; kt += 3) {
        FP4Q_GEMM_STEP(kt, st0, st1, st2, kt + NSTAGE - 1 < ksteps, kt + 1 == ksteps);
        if (kt + 1 < ksteps)
            FP4Q_GEMM_STEP(kt + 1, st1, st2, st0, kt + NSTAGE < ksteps, kt + 2 == ksteps);
        if (kt + 2 < ksteps)
            FP4Q_GEMM_STEP(kt + 2, st2, st0, st1, kt + NSTAGE + 1 < ksteps, kt + 3 == ksteps);
    }
#endif
#else
    // Register-staged pipeline: the loads of step t+3 are issued during
    // step t into registers and written to their LDS stage during step t+1,
    // so each load has a full step to arrive; the compiler tracks the
    // register dependencies (no LDS-DMA aliasing to reason about).
    StepRegs R;
    load_step<BF16OPS>(src, 0, R);
    store_step<BF16OPS>(R, st0, wave, lane);
    if (ksteps > 1) {
        load_step<BF16OPS>(src, 1, R);
        store_step<BF16OPS>(R, st1, wave, lane);
    }
    if (ksteps > 2) load_step<BF16OPS>(src, 2, R);
    __syncthreads();
    Frags FA, FB;
    uint32_t sa[4] = {0, 0, 0, 0}, sb[4] = {0, 0, 0, 0}, sa_n[4] = {0, 0, 0, 0},
             sb_n[4] = {0, 0, 0, 0};
    if (!BF16OPS) read_scales(st0, wm, wn, lane, sa, sb);
    read_frags(st0, 0, wm, wn, lane, FA);

#define FP4Q_GEMM_STEP(t, CUR, NEXT1, NEXTL, ISSUE, LAST)                          \
    do {                                                                           \
        read_frags(CUR, 1, wm, wn, lane, FB);                                      \
        mfma_half<BF16OPS>(FA, sa, sb, 0, acc);                                    \
        if ((t) + 2 < ksteps) store_step<BF16OPS>(R, NEXTL, wave, lane);           \
        if ((t) + 3 < ksteps) load_step<BF16OPS>(src, (t) + 3, R);                 \
        __builtin_amdgcn_sched_barrier(0);                                         \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                        \
        __builtin_amdgcn_s_barrier();                                              \
        __builtin_amdgcn_sched_barrier(0);                                         \
        if (!(LAST)) {                                                             \
            if (!BF16OPS) read_scales(NEXT1, wm, wn, lane, sa_n, sb_n);            \
            read_frags(NEXT1, 0, wm, wn, lane, FA);                                \
        }                                                                          \
        mfma_half<BF16OPS>(FB, sa, sb, 1, acc);                                    \
        _Pragma("unroll") for (int q = 0; q < 4; ++q) {                            \
            sa[q] = sa_n[q];                                                       \
            sb[q] = sb_n[q];                                                       \
        }                                                                          \
    } while (0)

    int kt = 0;
    for (; kt + 2 + 3 < ksteps; kt += 3) {
        FP4Q_GEMM_STEP(kt, st0, st1, st2, true, false);
        FP4Q_GEMM_STEP(kt + 1, st1, st2, st0, true, false);
        FP4Q_GEMM_STEP(kt + 2, st2, st0, st1, true, false);
    }
    for (; kt < ksteps; kt += 3) {
        FP4Q_GEMM_STEP(kt, st0, st1, st2, true, kt + 1 == ksteps);
        if (kt + 1 < ksteps) FP4Q_GEMM_STEP(kt + 1, st1, st2, st0, true, kt + 2 == ksteps);
        if (kt + 2 < ksteps) FP4Q_GEMM_STEP(kt + 2, st2, st0, st1, true, kt + 3 == ksteps);
    }
#endif
#undef FP4Q_GEMM_STEP

    // ---- epilogue: through LDS, so every lane writes 16 contiguous bytes ----
    // Each wave stages its 128 x 128 sub-tile 32 rows at a time in a private
    // LDS region (row pitch padded by 16 bytes), then reads it back as
    // 16-byte row chunks: 16 lanes cover one 128-column row.
    __syncthreads();  // all waves are done with the operand stages
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int PITCH = 128 * ESZ + 16;
    uint8_t* reg = OUT_BF16 ? st0 + wave * (32 * PITCH)
                            : (wave < 2 ? st0 : st1) + (wave & 1) * (32 * PITCH);
    const int row0 = m0 + wm * 128;
    const int col0 = n0 + wn * 128;
    const bool vec_ok = ((ldc * ESZ) % 16 == 0) && (((uintptr_t)cptr & 15) == 0);
    constexpr int CHUNK_ELEMS = 16 / ESZ;       // elements per 16-byte chunk
    constexpr int LANES_PER_ROW = 128 / CHUNK_ELEMS;
    constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = 8 * (r >> 2) + 4 * half + (r & 3);
                const int cl = j * 32 + l32;
                if (OUT_BF16)
                    *(uint16_t*)(reg + rl * PITCH + cl * 2) = (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
                else
                    *(float*)(reg + rl * PITCH + cl * 4) = acc[i][j][r];
            }
        __builtin_amdgcn_s_waitcnt(0xC07F);  // lgkmcnt(0): this wave's LDS writes done
        __builtin_amdgcn_wave_barrier();
        const int rbase = row0 + i * 32;
#pragma unroll
        for (int p = 0; p < 32 / ROWS_PER_PASS; ++p) {
            const int rl = p * ROWS_PER_PASS + lane / LANES_PER_ROW;
            const int ce = (lane % LANES_PER_ROW) * CHUNK_ELEMS;
            const uint4 v = *(const uint4*)(reg + rl * PITCH + ce * ESZ);
            const int row = rbase + rl;
            const int col = col0 + ce;
            if (row >= M) continue;
            const int64_t off = (int64_t)row * ldc + col;
            if (vec_ok && col + CHUNK_ELEMS <= N) {
                if (ACCUM) {
                    float4 o = *(const float4*)((const float*)cptr + off);
                    o.x += as_f32(v.x);
                    o.y += as_f32(v.y);
                    o.z += as_f32(v.z);
                    o.w += as_f32(v.w);
                    *(float4*)((float*)cptr + off) = o;
                } else if (OUT_BF16) {
                    *(uint4*)((uint16_t*)cptr + off) = v;
                } else {
                    *(uint4*)((float*)cptr + off) = v;
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

hipError_t launch_gemm_fp4(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                           const uint8_t* as, const uint8_t* bc, const uint8_t* bs, void* c,
                           int cdtype, int64_t ldc, bool accumulate, hipStream_t s) {
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    dim3 grid((unsigned)(tiles_m * tiles_n));
    if (cdtype == BF16)
        gemm_fp4_kernel<1, 0, 0><<<grid, kThreads, 0, s>>>((int)M, (int)N, (int)K, ac, as, bc, bs,
                                                           c, ldc, tiles_m, tiles_n);
    else if (accumulate)
        gemm_fp4_kernel<0, 1, 0><<<grid, kThreads, 0, s>>>((int)M, (int)N, (int)K, ac, as, bc, bs,
                                                           c, ldc, tiles_m, tiles_n);
    else
        gemm_fp4_kernel<0, 0, 0><<<grid, kThreads, 0, s>>>((int)M, (int)N, (int)K, ac, as, bc, bs,
                                                           c, ldc, tiles_m, tiles_n);
    return hipGetLastError();
}

hipError_t launch_gemm_bf16_accum(int64_t M, int64_t N, int64_t K, const uint16_t* a,
                                  const uint16_t* b, float* c, int64_t ldc, hipStream_t s) {
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    dim3 grid((unsigned)(tiles_m * tiles_n));
    gemm_fp4_kernel<0, 1, 1><<<grid, kThreads, 0, s>>>((int)M, (int)N, (int)K, (const uint8_t*)a,
                                                       nullptr, (const uint8_t*)b, nullptr, c, ldc,
                                                       tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace fp4q
