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
// Tiling: a workgroup of 2 x WN waves computes a 256 x 256 tile of C; each
// wave owns 128 rows x (256 / WN) columns as 4 x TN MFMA tiles.  With WN = 4
// (8 waves, 128 accumulator registers each) two waves share every SIMD, so
// one wave's MFMAs run while the other waits on LDS or the barrier.  The K
// loop steps 64 bytes per operand row (128 FP4 or 32 bf16 elements).
//
// Loads are coalesced: four consecutive lanes read one row's 64 bytes of
// the step (buffer loads against per-tile ranges, so rows past M or N read
// as zero), and are written to LDS in MFMA fragment order (fragment = 32
// rows x 32 bytes, 16 bytes per lane), with the 16-byte slot XOR-swizzled by
// the lane half and the fragment half so that both these writes and the
// MFMA-side 16-byte reads are free of bank conflicts.  A 3-stage LDS ring
// keeps two steps resident ahead of the one being computed: a step's loads
// are issued three steps early into registers and written to LDS one step
// later.  Scale words (4 bytes per row per step) travel with the codes.  The
// epilogue stages each wave's tile in LDS so every lane writes 16
// contiguous bytes.  Workgroups are remapped so that consecutive tiles of a
// grouped (4 tile-rows) order run on the same XCD and share its L2.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v16f __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
// Native 4 x 32-bit vectors (HIP's uint4 is a class with unions, which the
// compiler does not always split into registers).
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

static constexpr int BM = 256, BN = 256;
static constexpr int BKB = 64;                  // operand bytes per row per K step
static constexpr int FRAG = 1024;               // bytes per LDS fragment
static constexpr int OFF_B = 16 * FRAG;         // B fragments within a stage
static constexpr int OFF_SA = 32 * FRAG;        // A scale words (256 x 4 B)
static constexpr int OFF_SB = 32 * FRAG + 1024; // B scale words
static constexpr int STAGE = 32 * FRAG + 2048;
static constexpr int GROUP_M = 4;
static constexpr int BUF_FLAGS = 0x00020000;    // buffer resource word 3: raw 32-bit data
#ifndef FP4Q_GEMM_WN
#define FP4Q_GEMM_WN 4
#endif

template <int WN>
struct Layout {
    static constexpr int WAVES = 2 * WN;
    static constexpr int THREADS = 64 * WAVES;
    static constexpr int TN = 8 / WN;          // 32-column MFMA tiles per wave
    static constexpr int WCOLS = 32 * TN;      // columns per wave
    static constexpr int LPO = 16 / WAVES;     // 16-row load slices per operand per wave
    static constexpr int SPW = 8 / WAVES;      // scale words per lane per step
};

// 16-byte slot of (row r in 0..31, lane half h, fragment half kk) within a
// fragment: the MFMA lane h*32 + r, XOR-swizzled in bits 2 and 3.  A 16-lane
// LDS access group then covers 16 distinct slots both when lanes are
// (4 rows x 4 chunks of a row) and when they are 16 consecutive MFMA lanes.
__device__ __forceinline__ int frag_slot(int r, int h, int kk) {
    return (h * 32 + r) ^ (h << 2) ^ (kk << 3);
}

// Load sources: buffer resources whose ranges end at the operand's last row
// inside this tile (rows past M or N read as zero), per-slice row offsets of
// this lane (32-bit; they alone decide whether a row is in range), and the
// scalar byte offset of the current K step.
template <int WN>
struct Src {
    __amdgpu_buffer_rsrc_t ra, rb, rs0, rs1;  // rs1: second scale word (4-wave layout)
    uint32_t vrow[Layout<WN>::LPO];
    uint32_t vs[Layout<WN>::SPW];
    int soff, soff_s;
};

template <int WN>
struct StepRegs {
    u32x4 a[Layout<WN>::LPO], b[Layout<WN>::LPO];
    uint32_t s[Layout<WN>::SPW];
};

// Loads the K step the sources point at into registers and advances them.
template <int WN, int BF16OPS>
__device__ __forceinline__ void load_step(Src<WN>& src, StepRegs<WN>& R) {
    using L = Layout<WN>;
#pragma unroll
    for (int q = 0; q < L::LPO; ++q) {
        R.a[q] = __builtin_amdgcn_raw_buffer_load_b128(src.ra, src.vrow[q], src.soff, 0);
        R.b[q] = __builtin_amdgcn_raw_buffer_load_b128(src.rb, src.vrow[q], src.soff, 0);
    }
    if (!BF16OPS) {
#pragma unroll
        for (int j = 0; j < L::SPW; ++j)
            R.s[j] = __builtin_amdgcn_raw_buffer_load_b32(j == 0 ? src.rs0 : src.rs1, src.vs[j],
                                                          src.soff_s, 0);
    }
    src.soff += BKB;
    src.soff_s += 4;
}

// Writes a loaded step into `stage`: slice q of wave w is rows
// (q*WAVES + w)*16 .. +15; `lds_lane` is this lane's swizzled offset within
// a slice (chunk c = lane % 4 of row lane / 4 goes to fragment half c / 2,
// lane half c % 2).
template <int WN, int BF16OPS>
__device__ __forceinline__ void store_step(const StepRegs<WN>& R, uint8_t* stage, int wave,
                                           int lane, int lds_lane) {
    using L = Layout<WN>;
#pragma unroll
    for (int q = 0; q < L::LPO; ++q) {
        const int idx = q * L::WAVES + wave;
        const int off = (idx >> 1) * (2 * FRAG) + (idx & 1) * 256 + lds_lane;
        *(u32x4*)(stage + off) = R.a[q];
        *(u32x4*)(stage + OFF_B + off) = R.b[q];
    }
    if (!BF16OPS) {
        // scale word j of this lane belongs to combined row index
        // (j * WAVES + wave) * 64 + lane: A rows 0..255, then B rows
#pragma unroll
        for (int j = 0; j < L::SPW; ++j)
            *(uint32_t*)(stage + OFF_SA + ((j * L::WAVES + wave) * 64 + lane) * 4) = R.s[j];
    }
}

template <int WN>
struct Frags {
    u32x4 a[4], b[Layout<WN>::TN];
};

// This wave's A and B fragments of half kk of a staged step.
template <int WN>
__device__ __forceinline__ void read_frags(const uint8_t* base, int kk, int wm, int wn, int lane,
                                           Frags<WN>& F) {
    using L = Layout<WN>;
    const int slot = frag_slot(lane & 31, lane >> 5, kk) * 16;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        F.a[i] = *(const u32x4*)(base + ((wm * 4 + i) * 2 + kk) * FRAG + slot);
#pragma unroll
    for (int j = 0; j < L::TN; ++j)
        F.b[j] = *(const u32x4*)(base + OFF_B + ((wn * L::TN + j) * 2 + kk) * FRAG + slot);
}

// Scale words (4 K blocks of 32 elements each) of this lane's MFMA rows (A)
// and columns (B).
template <int WN>
__device__ __forceinline__ void read_scales(const uint8_t* base, int wm, int wn, int lane,
                                            uint32_t (&sa)[4], uint32_t (&sb)[Layout<WN>::TN]) {
    using L = Layout<WN>;
    const int l32 = lane & 31;
#pragma unroll
    for (int i = 0; i < 4; ++i)
        sa[i] = *(const uint32_t*)(base + OFF_SA + (wm * 128 + i * 32 + l32) * 4);
#pragma unroll
    for (int j = 0; j < L::TN; ++j)
        sb[j] = *(const uint32_t*)(base + OFF_SB + (wn * L::WCOLS + j * 32 + l32) * 4);
}

// Shifts raw scale words so that byte 2 kk is the K block of half kk for
// this lane's 32-element K chunk (lanes 32..63 take the odd blocks).
template <int WN>
__device__ __forceinline__ void shift_scales(const uint32_t (&ra)[4],
                                             const uint32_t (&rb)[Layout<WN>::TN], int sh,
                                             uint32_t (&sa)[4], uint32_t (&sb)[Layout<WN>::TN]) {
#pragma unroll
    for (int i = 0; i < 4; ++i) sa[i] = ra[i] >> sh;
#pragma unroll
    for (int j = 0; j < Layout<WN>::TN; ++j) sb[j] = rb[j] >> sh;
}

// The 4 x TN MFMAs of this wave on half KK of a K step.  FP4: the scaled
// MFMA on E2M1 operands (64 K elements per half), its byte select picking
// byte 2 KK of the lane's (pre-shifted) scale words; BF16: plain bf16 MFMAs
// (16 K elements per half, the same 16 bytes per lane).
template <int WN, int BF16OPS, int KK>
__device__ __forceinline__ void mfma_half(const Frags<WN>& F, const uint32_t (&sa)[4],
                                          const uint32_t (&sb)[Layout<WN>::TN],
                                          v16f (&acc)[4][Layout<WN>::TN]) {
    using L = Layout<WN>;
    if (BF16OPS) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int j = 0; j < L::TN; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(
                    __builtin_bit_cast(bf16x8_t, F.a[i]), __builtin_bit_cast(bf16x8_t, F.b[j]),
                    acc[i][j], 0, 0, 0);
        return;
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const v8i fa = (v8i){(int)F.a[i].x, (int)F.a[i].y, (int)F.a[i].z, (int)F.a[i].w, 0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < L::TN; ++j) {
            const v8i fb =
                (v8i){(int)F.b[j].x, (int)F.b[j].y, (int)F.b[j].z, (int)F.b[j].w, 0, 0, 0, 0};
            acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                fa, fb, acc[i][j], 4, 4, 2 * KK, (int)sa[i], 2 * KK, (int)sb[j]);
        }
    }
}

template <int WN, int OUT_BF16, int ACCUM, int BF16OPS>
__global__ __launch_bounds__(Layout<WN>::THREADS, 1) void gemm_fp4_kernel(
    int M, int N, int K, const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, void* __restrict__ cptr,
    int64_t ldc, int tiles_m, int tiles_n) {
#if defined(__HIP_DEVICE_COMPILE__)  // the host pass cannot instantiate buffer resources
    using L = Layout<WN>;
    constexpr int TN = L::TN;
    // The LDS ring stages are separate objects; the epilogue reuses them.
    __shared__ __attribute__((aligned(16))) uint8_t st0[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st1[STAGE];
    __shared__ __attribute__((aligned(16))) uint8_t st2[STAGE];

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
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int half = lane >> 5;
    const int l32 = lane & 31;
    // bytes per operand row (< 2^23, checked by the caller); each K step
    // consumes 64 of them
    const int kbytes = BF16OPS ? K * 2 : K / 2;
    const int kscale = K / 32;
    const int ksteps = kbytes / BKB;

    Src<WN> src;
    {
        const int rows_a = min(M - m0, BM), rows_b = min(N - n0, BN);
        src.ra = __builtin_amdgcn_make_buffer_rsrc((void*)(ac + (int64_t)m0 * kbytes), (short)0,
                                                   rows_a * kbytes, BUF_FLAGS);
        src.rb = __builtin_amdgcn_make_buffer_rsrc((void*)(bc + (int64_t)n0 * kbytes), (short)0,
                                                   rows_b * kbytes, BUF_FLAGS);
#pragma unroll
        for (int q = 0; q < L::LPO; ++q)
            src.vrow[q] = (uint32_t)(((q * L::WAVES + wave) * 16 + (lane >> 2)) * kbytes +
                                     (lane & 3) * 16);
        const __amdgpu_buffer_rsrc_t rsa = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(as + (int64_t)m0 * kscale), (short)0, rows_a * kscale, BUF_FLAGS);
        const __amdgpu_buffer_rsrc_t rsb = __builtin_amdgcn_make_buffer_rsrc(
            (void*)(bs + (int64_t)n0 * kscale), (short)0, rows_b * kscale, BUF_FLAGS);
#pragma unroll
        for (int j = 0; j < L::SPW; ++j) {
            const int cw = j * L::WAVES + wave;  // combined row / 64: A rows, then B rows
            if (j == 0)
                src.rs0 = cw < 4 ? rsa : rsb;
            else
                src.rs1 = cw < 4 ? rsa : rsb;
            src.vs[j] = (uint32_t)(((cw & 3) * 64 + lane) * kscale);
        }
        src.soff = 0;
        src.soff_s = 0;
    }
    // this lane's chunk c = lane % 4 of row lane / 4 in a 16-row slice
    const int lds_lane = ((lane & 3) >> 1) * FRAG +
                         frag_slot(lane >> 2, lane & 1, (lane & 3) >> 1) * 16;

    v16f acc[4][TN];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    Frags<WN> FA, FB;
    // sa/sb: shifted scale words of the step being computed; ra/rb: raw
    // words of the next step, read after the barrier that publishes it.
    uint32_t sa[4] = {0, 0, 0, 0}, ra[4] = {0, 0, 0, 0};
    uint32_t sb[TN], rb[TN];
#pragma unroll
    for (int j = 0; j < TN; ++j) sb[j] = rb[j] = 0;
    const int sh = 8 * half;

    // Software pipeline over K steps t, LDS ring of 3 stages: the loads of
    // step t + 3 are issued in step t into registers and written to their
    // stage in step t + 1.  Each step computes two halves (K bytes 0..31 and
    // 32..63 of the step); order within a step, fenced against the
    // compiler's scheduler:
    //   1. shift the step's scale words; read the fragments of (t, 1);
    //   2. MFMAs of (t, 0), whose fragments were read during step t - 1;
    //      write the registers loaded during step t - 1 (step t + 2) to the
    //      stage that step t - 1 used; issue the loads of step t + 3;
    //   3. lgkmcnt(0) (this wave's LDS traffic), then one workgroup barrier,
    //      which orders those writes and every wave's reads of that stage;
    //   4. read the scales and (t + 1, 0) fragments; MFMAs of (t, 1).
    // LDS reads thus always run under MFMAs of the other half.
    StepRegs<WN> R;
    load_step<WN, BF16OPS>(src, R);
    store_step<WN, BF16OPS>(R, st0, wave, lane, lds_lane);
    if (ksteps > 1) {
        load_step<WN, BF16OPS>(src, R);
        store_step<WN, BF16OPS>(R, st1, wave, lane, lds_lane);
    }
    if (ksteps > 2) load_step<WN, BF16OPS>(src, R);
    __syncthreads();
    if (!BF16OPS) read_scales<WN>(st0, wm, wn, lane, ra, rb);
    read_frags<WN>(st0, 0, wm, wn, lane, FA);

// LAST is 2 in the steady-state loop (every later step exists, so the
// step's loads are unconditional), else whether t is the final step.
#define FP4Q_GEMM_STEP(t, CUR, NEXT1, NEXTL, LAST)                                 \
    do {                                                                           \
        __builtin_amdgcn_sched_barrier(0);                                         \
        if (!BF16OPS) shift_scales<WN>(ra, rb, sh, sa, sb);                        \
        read_frags<WN>(CUR, 1, wm, wn, lane, FB);                                  \
        __builtin_amdgcn_sched_barrier(0);                                         \
        mfma_half<WN, BF16OPS, 0>(FA, sa, sb, acc);                                \
        if ((LAST) == 2 || (t) + 2 < ksteps)                                       \
            store_step<WN, BF16OPS>(R, NEXTL, wave, lane, lds_lane);               \
        if ((LAST) == 2 || (t) + 3 < ksteps) load_step<WN, BF16OPS>(src, R);       \
        __builtin_amdgcn_sched_barrier(0);                                         \
        __builtin_amdgcn_s_waitcnt(0xC07F);                                        \
        __builtin_amdgcn_s_barrier();                                              \
        __builtin_amdgcn_sched_barrier(0);                                         \
        if ((LAST) != 1) {                                                         \
            if (!BF16OPS) read_scales<WN>(NEXT1, wm, wn, lane, ra, rb);            \
            read_frags<WN>(NEXT1, 0, wm, wn, lane, FA);                            \
        }                                                                          \
        mfma_half<WN, BF16OPS, 1>(FB, sa, sb, acc);                                \
    } while (0)

    // The ring position of step t is t % 3; NEXTL is the stage written
    // during step t (the one step t - 1 used).
    int kt = 0;
    for (; kt + 2 + 3 < ksteps; kt += 3) {
        FP4Q_GEMM_STEP(kt, st0, st1, st2, 2);
        FP4Q_GEMM_STEP(kt + 1, st1, st2, st0, 2);
        FP4Q_GEMM_STEP(kt + 2, st2, st0, st1, 2);
    }
    for (; kt < ksteps; kt += 3) {
        FP4Q_GEMM_STEP(kt, st0, st1, st2, kt + 1 == ksteps);
        if (kt + 1 < ksteps) FP4Q_GEMM_STEP(kt + 1, st1, st2, st0, kt + 2 == ksteps);
        if (kt + 2 < ksteps) FP4Q_GEMM_STEP(kt + 2, st2, st0, st1, kt + 3 == ksteps);
    }
#undef FP4Q_GEMM_STEP

    // ---- epilogue: through LDS, so every lane writes 16 contiguous bytes ----
    // Each wave stages its tile 32 rows at a time in a private LDS region
    // (row pitch padded by 16 bytes), then reads it back as 16-byte row
    // chunks.
    __syncthreads();  // all waves are done with the operand stages
    constexpr int ESZ = OUT_BF16 ? 2 : 4;
    constexpr int PITCH = L::WCOLS * ESZ + 16;
    constexpr int REGION = 32 * PITCH;
    constexpr int PER_STAGE = STAGE / REGION;  // wave regions that fit in one stage
    uint8_t* reg = (wave / PER_STAGE == 0 ? st0 : wave / PER_STAGE == 1 ? st1 : st2) +
                   (wave % PER_STAGE) * REGION;
    const int row0 = m0 + wm * 128;
    const int col0 = n0 + wn * L::WCOLS;
    const bool vec_ok = ((ldc * ESZ) % 16 == 0) && (((uintptr_t)cptr & 15) == 0);
    constexpr int CHUNK_ELEMS = 16 / ESZ;  // elements per 16-byte chunk
    constexpr int LANES_PER_ROW = L::WCOLS / CHUNK_ELEMS;
    constexpr int ROWS_PER_PASS = 64 / LANES_PER_ROW;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < TN; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int rl = 8 * (r >> 2) + 4 * half + (r & 3);
                const int cl = j * 32 + l32;
                if (OUT_BF16)
                    *(uint16_t*)(reg + rl * PITCH + cl * 2) =
                        (uint16_t)f32_to_bf16_bits(acc[i][j][r]);
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
            const u32x4 v = *(const u32x4*)(reg + rl * PITCH + ce * ESZ);
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
                    *(u32x4*)((uint16_t*)cptr + off) = v;
                } else {
                    *(u32x4*)((float*)cptr + off) = v;
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
#endif
}

template <int OUT_BF16, int ACCUM, int BF16OPS>
static void launch_tiles(int64_t M, int64_t N, int64_t K, const uint8_t* a, const uint8_t* as,
                         const uint8_t* b, const uint8_t* bs, void* c, int64_t ldc,
                         hipStream_t s) {
    constexpr int WN = FP4Q_GEMM_WN;
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    gemm_fp4_kernel<WN, OUT_BF16, ACCUM, BF16OPS>
        <<<dim3((unsigned)(tiles_m * tiles_n)), Layout<WN>::THREADS, 0, s>>>(
            (int)M, (int)N, (int)K, a, as, b, bs, c, ldc, tiles_m, tiles_n);
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

}  // namespace fp4q
