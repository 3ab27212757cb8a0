// On-device choice of the hot channels: the outlier-dynamics page (sec. 4.1)
// keeps the top 9% of channels, ranked by quantisation error, in high
// precision.  Here the error of channel (column) c of X [M, K] is
//
//   e_c = sum_i ( x_ic - deq(Q(x))_ic )^2
//
// with Q the ROW block-32 nearest-even quantisation the forward GEMM uses;
// the n_hot channels of largest e_c are returned in ascending index order
// (ties: the lower index first; a NaN error ranks above every number).
//
// Kernels:
//  * hot_err_partial: a workgroup of 4 waves owns a slab of rows (a multiple
//    of 64, chosen per shape so the grid fills the chip) x 512 columns; a lane
//    owns 8 adjacent columns (four adjacent lanes = one 32-column block, the
//    block maximum by DPP), quantises and dequantises each of its rows with
//    the hardware scaled converts, and accumulates the squared error; the
//    four waves' sums meet in LDS in a fixed order and one partial row per
//    slab is written (no atomics: the result does not depend on the order
//    workgroups run in).
//  * hot_err_final: per column, the slabs' partials summed in a fixed order
//    (eight waves take interleaved slabs, then combine in LDS).
//  * hot_select: one workgroup of 1024 threads holding all (<= 16384)
//    errors in registers, 16 consecutive channels per thread: a 4-pass
//    radix select (8-bit digits, LDS histograms) finds the n-th largest
//    error bit pattern T; the channels above T, and the lowest-index ones
//    equal to T, are compacted in index order by two block-wide prefix sums.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

static constexpr int kErrThreads = 256;
static constexpr int kErrRows = 64;     // slab granularity (rows)
static constexpr int kErrCols = 512;    // columns per workgroup (8 per lane)
static constexpr int kSelThreads = 1024;
static constexpr int kSelPer = 16;      // channels per selection thread
static constexpr int kSelMax = kSelThreads * kSelPer;

// Squared-error sums of one row's 8 columns (one bf16 uint4) into acc.
__device__ __forceinline__ void err_row(uint4 v, float acc[8]) {
    const uint32_t w0 = v.x, w1 = v.y, w2 = v.z, w3 = v.w;
    const u16x2_t m0 = __builtin_bit_cast(u16x2_t, w0 & 0x7FFF7FFFu);
    const u16x2_t m1 = __builtin_bit_cast(u16x2_t, w1 & 0x7FFF7FFFu);
    const u16x2_t m2 = __builtin_bit_cast(u16x2_t, w2 & 0x7FFF7FFFu);
    const u16x2_t m3 = __builtin_bit_cast(u16x2_t, w3 & 0x7FFF7FFFu);
    const u16x2_t mm = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1),
                                                 __builtin_elementwise_max(m2, m3));
    const uint32_t amax = group_max_u32<4>(((uint32_t)max(mm.x, mm.y)) << 16);
    const bool nonfinite = amax >= 0x7F800000u;
    const float sc = e8m0_scale_f32(nonfinite ? 0u : e8m0_from_amax(amax));
    uint32_t packed = 0;
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w0), sc, 0);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w1), sc, 1);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w2), sc, 2);
    packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w3), sc, 3);
    // dequantised pairs, exact in fp32; x - deq is exact too (both lie within
    // a few binades of the block scale), so only the square and sum round
    const f32x2_t d0 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, sc, 0);
    const f32x2_t d1 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, sc, 1);
    const f32x2_t d2 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, sc, 2);
    const f32x2_t d3 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(packed, sc, 3);
    const float q[8] = {d0.x, d0.y, d1.x, d1.y, d2.x, d2.y, d3.x, d3.y};
    const float xv[8] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1),
                         bf16_lo(w2), bf16_hi(w2), bf16_lo(w3), bf16_hi(w3)};
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        const float e = nonfinite ? __builtin_nanf("") : xv[j] - q[j];
        acc[j] += e * e;
    }
}

__global__ __launch_bounds__(kErrThreads) void hot_err_partial(const uint16_t* __restrict__ x,
                                                               int64_t rows, int64_t cols,
                                                               int64_t ld, int slab,
                                                               float* __restrict__ partial) {
    __shared__ float red[4][kErrCols];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c0 = (int64_t)blockIdx.y * kErrCols + lane * 8;
    const bool cok = c0 < cols;  // cols % 32 == 0: a block is wholly in or out
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    const int64_t rbeg = (int64_t)blockIdx.x * slab;
    const int64_t rend = min(rows, rbeg + slab);
    const uint16_t* p = x + c0;
    // rows rbeg + wave + 4t; four loads in flight before their arithmetic
    int64_t r = rbeg + wave;
    for (; r + 12 < rend; r += 16) {
        uint4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
            v[u] = cok ? *(const uint4*)(p + (r + 4 * u) * ld) : make_uint4(0u, 0u, 0u, 0u);
#pragma unroll
        for (int u = 0; u < 4; ++u) err_row(v[u], acc);
    }
    for (; r < rend; r += 4) {
        const uint4 v = cok ? *(const uint4*)(p + r * ld) : make_uint4(0u, 0u, 0u, 0u);
        err_row(v, acc);
    }
#pragma unroll
    for (int j = 0; j < 8; ++j) red[wave][lane * 8 + j] = acc[j];
    __syncthreads();
    for (int c = threadIdx.x; c < kErrCols; c += kErrThreads) {
        const int64_t col = (int64_t)blockIdx.y * kErrCols + c;
        if (col < cols)
            partial[(int64_t)blockIdx.x * cols + col] = ((red[0][c] + red[1][c]) + red[2][c]) + red[3][c];
    }
}

// 64 columns per workgroup of 8 waves; wave w sums slabs w, w + 8, ... in
// order (eight loads in flight), then the eight sums are added in wave order.
static constexpr int kFinThreads = 512;
__global__ __launch_bounds__(kFinThreads) void hot_err_final(const float* __restrict__ partial,
                                                             int64_t tiles, int64_t cols,
                                                             float* __restrict__ err) {
    __shared__ float red[8][64];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int64_t c = (int64_t)blockIdx.x * 64 + lane;
    float s = 0.f;
    if (c < cols) {
        int64_t t = wave;
        for (; t + 56 < tiles; t += 64) {
            float v[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) v[u] = partial[(t + 8 * u) * cols + c];
#pragma unroll
            for (int u = 0; u < 8; ++u) s += v[u];
        }
        for (; t < tiles; t += 8) s += partial[t * cols + c];
    }
    red[wave][lane] = s;
    __syncthreads();
    if (wave == 0 && c < cols) {
        float r = red[0][lane];
#pragma unroll
        for (int w = 1; w < 8; ++w) r += red[w][lane];
        err[c] = r;
    }
}

__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t t = __shfl_up(v, d, 64);
        if (lane >= d) v += t;
    }
    return v;
}

// Exclusive prefix sum of v over the workgroup's threads in thread order
// (blockDim.x = 1024).  wtot: 16 words of LDS; ends with a barrier.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* wtot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t inc = wave_incl_scan(v, lane);
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    uint32_t base = 0;
    for (int w = 0; w < wave; ++w) base += wtot[w];
    __syncthreads();
    return base + inc - v;
}

// Errors as ordered bit patterns: every e_c >= 0 or NaN; the fp32 bits of
// non-negative numbers order as their values and NaN is given 0x7FFFFFFF,
// above +inf.
__global__ __launch_bounds__(kSelThreads) void hot_select(const float* __restrict__ err,
                                                          int cols, int n_hot,
                                                          int32_t* __restrict__ hot) {
    __shared__ uint32_t hist[256];
    __shared__ uint32_t wtot[16];
    __shared__ uint32_t found[2];
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int base = tid * kSelPer;
    uint32_t eb[kSelPer];
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
        const int i = base + j;
        uint32_t b = 0;
        if (i < cols) {
            const float e = err[i];
            b = e != e ? 0x7FFFFFFFu : as_u32(e);
        }
        eb[j] = b;
    }
    // radix select of the n_hot-th largest pattern, most significant digit
    // first; `need` is its rank among the patterns that share the prefix
    uint32_t prefix = 0, mask = 0, need = (uint32_t)n_hot;
    for (int shift = 24; shift >= 0; shift -= 8) {
        if (tid < 256) hist[tid] = 0;
        __syncthreads();
        // runs of equal digits among a thread's consecutive channels go in as
        // one add (errors of one magnitude share their leading digits, and
        // same-address LDS atomics serialise)
        uint32_t cur = 0, cnt = 0;
#pragma unroll
        for (int j = 0; j < kSelPer; ++j) {
            if (base + j < cols && (eb[j] & mask) == prefix) {
                const uint32_t d = (eb[j] >> shift) & 255u;
                if (cnt && d != cur) {
                    atomicAdd(&hist[cur], cnt);
                    cnt = 0;
                }
                cur = d;
                ++cnt;
            }
        }
        if (cnt) atomicAdd(&hist[cur], cnt);
        __syncthreads();
        // counts at or above each digit: threads 0..255 take the digits in
        // descending order (thread t -> digit 255 - t), an inclusive scan
        uint32_t h = 0, inc = 0;
        if (tid < 256) {
            h = hist[255 - tid];
            inc = wave_incl_scan(h, lane);
            if (lane == 63) wtot[wave] = inc;
        }
        __syncthreads();
        if (tid < 256) {
            for (int w = 0; w < wave; ++w) inc += wtot[w];
            if (inc >= need && inc - h < need) {  // exactly one digit
                found[0] = 255u - (uint32_t)tid;
                found[1] = inc - h;                // patterns above it
            }
        }
        __syncthreads();
        const uint32_t d = found[0];
        need -= found[1];
        prefix |= d << shift;
        mask |= 255u << shift;
        __syncthreads();
    }
    // T = prefix: take every pattern above T and the `need` lowest-index
    // channels equal to T
    uint32_t neq = 0;
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) neq += (base + j < cols && eb[j] == prefix) ? 1u : 0u;
    uint32_t eqrank = block_excl_scan(neq, wtot);
    uint32_t take = 0;
    uint32_t nsel = 0;
#pragma unroll
    for (int j = 0; j < kSelPer; ++j) {
        const bool ok = base + j < cols;
        bool s = ok && eb[j] > prefix;
        if (ok && eb[j] == prefix) {
            s = eqrank < need;
            ++eqrank;
        }
        take |= (s ? 1u : 0u) << j;
        nsel += s ? 1u : 0u;
    }
    uint32_t pos = block_excl_scan(nsel, wtot);
#pragma unroll
    for (int j = 0; j < kSelPer; ++j)
        if (take & (1u << j)) hot[pos++] = base + j;
}

size_t hot_channels_workspace_bytes(int64_t rows, int64_t cols) {
    const int64_t tiles = (rows + kErrRows - 1) / kErrRows;
    return (size_t)((tiles + 1) * cols) * sizeof(float);
}

int64_t hot_channels_max_cols() { return kSelMax; }

// Rows per slab: the largest power-of-two multiple of 64 (at most 1024) that
// still gives the partial pass at least 1024 workgroups (4 per compute unit,
// each lane with four 16-byte loads in flight), so the grid fills the chip
// and the final pass has few slabs to add.
static int64_t slab_rows(int64_t rows, int64_t cols) {
    const int64_t strips = (cols + kErrCols - 1) / kErrCols;
    int64_t slab = kErrRows;
    while (slab < 1024 && ((rows + 2 * slab - 1) / (2 * slab)) * strips >= 1024) slab *= 2;
    return slab;
}

hipError_t launch_hot_channels(const uint16_t* x, int64_t rows, int64_t cols, int64_t ld,
                               int32_t n_hot, void* ws, int32_t* hot, float* err_out,
                               hipStream_t s) {
    const int64_t slab = slab_rows(rows, cols);
    const int64_t tiles = (rows + slab - 1) / slab;
    float* partial = (float*)ws;
    float* err = err_out ? err_out : partial + tiles * cols;
    dim3 g1((unsigned)tiles, (unsigned)((cols + kErrCols - 1) / kErrCols));
    FP4Q_LAUNCH((hot_err_partial), g1, kErrThreads, 0, s, x, rows, cols, ld, (int)slab, partial);
    FP4Q_LAUNCH((hot_err_final), dim3((unsigned)((cols + 63) / 64)), kFinThreads, 0, s, partial, tiles, cols,
                                                                             err);
    if (n_hot > 0) FP4Q_LAUNCH((hot_select), 1, kSelThreads, 0, s, err, (int)cols, n_hot, hot);
    return hipGetLastError();
}

}  // namespace fp4q
