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

static constexpr int BM = 256, BN = 256;
static constexpr int BKB = 64;  // K bytes per step (128 fp4 elements)
static constexpr int kThreads = 256;
static constexpr int FRAG = 1024;                    // bytes per LDS fragment
static constexpr int STAGE = 2 * 16 * FRAG;          // A + B fragments per stage
static constexpr int GROUP_M = 4;

template <int OUT_BF16, int ACCUM>
__global__ __launch_bounds__(kThreads, 1) void gemm_fp4_kernel(
    int M, int N, int K, const uint8_t* __restrict__ ac, const uint8_t* __restrict__ as,
    const uint8_t* __restrict__ bc, const uint8_t* __restrict__ bs, void* __restrict__ cptr,
    int64_t ldc, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(16))) uint8_t lds[2 * STAGE];

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
    const int half = lane >> 5;  // which 16-byte half of a 32-byte fragment row
    const int l32 = lane & 31;
    const int64_t kbytes = K / 2;
    const int kscale = K / 32;
    const int ksteps = K / 128;

    // Global sources of this lane's 8 fragment loads per step: wave w loads
    // A fragments f = 4w..4w+3 and B fragments f = 4w..4w+3, f = rg*2 + kk.
    const uint8_t* ga[4];
    const uint8_t* gb[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int f = wave * 4 + q;
        const int rg = f >> 1, kk = f & 1;
        const int ra = min(m0 + rg * 32 + l32, M - 1);
        const int rb = min(n0 + rg * 32 + l32, N - 1);
        ga[q] = ac + (int64_t)ra * kbytes + kk * 32 + half * 16;
        gb[q] = bc + (int64_t)rb * kbytes + kk * 32 + half * 16;
    }
    // Scale rows this lane feeds to its MFMAs: A rows of the wave's 4 row
    // groups, B rows of its 4 column groups.
    const uint32_t* sa_ptr[4];
    const uint32_t* sb_ptr[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int ra = min(m0 + wm * 128 + i * 32 + l32, M - 1);
        const int rb = min(n0 + wn * 128 + i * 32 + l32, N - 1);
        sa_ptr[i] = (const uint32_t*)(as + (int64_t)ra * kscale);
        sb_ptr[i] = (const uint32_t*)(bs + (int64_t)rb * kscale);
    }

    v16f acc[4][4];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j)
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[i][j][r] = 0.0f;

    uint4 pa[4], pb[4];
    uint32_t sa_cur[4], sb_cur[4], sa_nxt[4], sb_nxt[4];

    auto gload = [&](int kt) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            pa[q] = *(const uint4*)(ga[q] + (int64_t)kt * BKB);
            pb[q] = *(const uint4*)(gb[q] + (int64_t)kt * BKB);
        }
    };
    auto sload = [&](int kt, uint32_t (&sa)[4], uint32_t (&sb)[4]) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sa[i] = sa_ptr[i][kt] >> (8 * half);
            sb[i] = sb_ptr[i][kt] >> (8 * half);
        }
    };
    auto lds_store = [&](int buf) {
        uint8_t* base = lds + buf * STAGE;
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int f = wave * 4 + q;
            *(uint4*)(base + f * FRAG + lane * 16) = pa[q];
            *(uint4*)(base + 16 * FRAG + f * FRAG + lane * 16) = pb[q];
        }
    };

    gload(0);
    sload(0, sa_cur, sb_cur);
    lds_store(0);
    __syncthreads();

    for (int kt = 0; kt < ksteps; ++kt) {
        const int buf = kt & 1;
        const bool more = kt + 1 < ksteps;
        if (more) {
            gload(kt + 1);
            sload(kt + 1, sa_nxt, sb_nxt);
        }
        const uint8_t* base = lds + buf * STAGE;
#pragma unroll
        for (int kk = 0; kk < 2; ++kk) {
            v8i fa[4], fb[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const uint4 a = *(const uint4*)(base + ((wm * 4 + i) * 2 + kk) * FRAG + lane * 16);
                const uint4 b =
                    *(const uint4*)(base + 16 * FRAG + ((wn * 4 + i) * 2 + kk) * FRAG + lane * 16);
                fa[i] = (v8i){(int)a.x, (int)a.y, (int)a.z, (int)a.w, 0, 0, 0, 0};
                fb[i] = (v8i){(int)b.x, (int)b.y, (int)b.z, (int)b.w, 0, 0, 0, 0};
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_scale_f32_32x32x64_f8f6f4(
                        fa[i], fb[j], acc[i][j], 4, 4, 0, (int)(sa_cur[i] >> (16 * kk)), 0,
                        (int)(sb_cur[j] >> (16 * kk)));
        }
        if (more) {
            lds_store(buf ^ 1);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                sa_cur[i] = sa_nxt[i];
                sb_cur[i] = sb_nxt[i];
            }
        }
        __syncthreads();
    }

    // ---- epilogue ----
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int col = n0 + wn * 128 + j * 32 + l32;
            if (col >= N) continue;
#pragma unroll
            for (int r = 0; r < 16; ++r) {
                const int row = m0 + wm * 128 + i * 32 + 8 * (r >> 2) + 4 * half + (r & 3);
                if (row < M) {
                    const int64_t off = (int64_t)row * ldc + col;
                    const float v = acc[i][j][r];
                    if (OUT_BF16) {
                        ((uint16_t*)cptr)[off] = (uint16_t)f32_to_bf16_bits(v);
                    } else if (ACCUM) {
                        ((float*)cptr)[off] += v;
                    } else {
                        ((float*)cptr)[off] = v;
                    }
                }
            }
        }
    }
}

hipError_t launch_gemm_fp4(int64_t M, int64_t N, int64_t K, const uint8_t* ac,
                           const uint8_t* as, const uint8_t* bc, const uint8_t* bs, void* c,
                           int cdtype, int64_t ldc, bool accumulate, hipStream_t s) {
    const int tiles_m = (int)((M + BM - 1) / BM);
    const int tiles_n = (int)((N + BN - 1) / BN);
    dim3 grid((unsigned)(tiles_m * tiles_n));
    if (cdtype == BF16)
        gemm_fp4_kernel<1, 0><<<grid, kThreads, 0, s>>>((int)M, (int)N, (int)K, ac, as, bc, bs, c,
                                                        ldc, tiles_m, tiles_n);
    else if (accumulate)
        gemm_fp4_kernel<0, 1><<<grid, kThreads, 0, s>>>((int)M, (int)N, (int)K, ac, as, bc, bs, c,
                                                        ldc, tiles_m, tiles_n);
    else
        gemm_fp4_kernel<0, 0><<<grid, kThreads, 0, s>>>((int)M, (int)N, (int)K, ac, as, bc, bs, c,
                                                        ldc, tiles_m, tiles_n);
    return hipGetLastError();
}

}  // namespace fp4q
