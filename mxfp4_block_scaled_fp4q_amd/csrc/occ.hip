// Outlier clamping and compensation (the MSRA FP4-training summary page,
// sec. 三 and 六): the activations' largest magnitudes are clamped to the
// tensor's `quantile` quantile T before the FP4 quantisation, and what the
// clamp removed is kept as a sparse high-precision residual whose product
// with the weight is added to the FP4 GEMM's output.
//
//   T        = the j-th smallest |x| over the tensor, j = ceil(quantile * n)
//              (an order statistic; NaN ranks above every number)
//   outlier  = |x| ranks above T (so NaN is an outlier while T is finite)
//   clamp(x) = sign(x) T on outliers, x elsewhere (exact in bf16)
//   R        = x - clamp(x) on outliers: CSR, columns ascending per row,
//              fp32 values (one correctly rounded fp32 subtraction)
//
// Kernels (fp4q_occ_quantize): bf16 has 2^15 magnitudes, so one histogram
// pass over |x| bit patterns gives T exactly:
//  * occ_zero: clears the histogram and the per-row counts (a fill kernel,
//    not a memset, so the call can be captured).
//  * occ_hist: one 1024-thread workgroup per compute unit streams x and
//    counts magnitudes in a 32768-bin LDS histogram (128 KB), then adds its
//    non-zero bins to the global histogram (integer atomics: order-free).
//  * occ_select: one workgroup prefix-sums the histogram and finds the bin
//    holding the j-th magnitude.
//  * occ_clamp_quant: the ROW block-32 quantiser on the clamped values
//    (nearest-even or stochastic, the ordinary counters), also writing one
//    mask bit per element and each row's outlier count.
//  * occ_scan: row counts -> int64 row pointers (one workgroup).
//  * occ_fill: a wave per row walks the row's mask bytes in order (a wave
//    prefix sum places each lane's outliers) and writes column and residual.
// fp4q_occ_spmm: Y[i, :] += sum over row i's entries (in CSR order) of
// R[i,k] W[k, :] (fp32, fused multiply-adds from zero in CSR order, then one
// add into Y), one workgroup per (row, 2048 columns); rows without outliers
// are not touched.
#include "fp4q_device.h"
#include "fp4q_internal.h"

namespace fp4q {

static constexpr int kOccBins = 32768;
static constexpr int kOccHistThreads = 1024;
static constexpr int kOccScanLds = 8192;  // rows whose scan is staged in LDS (8 per thread)
static constexpr int kOccThreads = 256;

struct OccWs {
    uint32_t* hist;     // [32768]
    uint32_t* params;   // [0] = T's bf16 magnitude bits
    uint32_t* row_cnt;  // [rows]
    uint8_t* mask;      // [rows, cols / 8]
};

static size_t align256(size_t v) { return (v + 255) & ~(size_t)255; }

static OccWs occ_ws(void* ws, int64_t rows) {
    uint8_t* p = (uint8_t*)ws;
    OccWs w;
    w.hist = (uint32_t*)p;
    p += align256(sizeof(uint32_t) * kOccBins);
    w.params = (uint32_t*)p;
    p += 256;
    w.row_cnt = (uint32_t*)p;
    p += align256(sizeof(uint32_t) * (size_t)rows);
    w.mask = p;
    return w;
}

size_t occ_workspace_bytes(int64_t rows, int64_t cols) {
    return align256(sizeof(uint32_t) * kOccBins) + 256 + align256(sizeof(uint32_t) * (size_t)rows) +
           align256((size_t)rows * (size_t)(cols / 8));
}

__global__ __launch_bounds__(kOccThreads) void occ_zero(uint32_t* hist, uint32_t* row_cnt,
                                                        int64_t rows) {
    const int64_t i = (int64_t)blockIdx.x * kOccThreads + threadIdx.x;
    if (i < kOccBins) hist[i] = 0;
    if (i < rows) row_cnt[i] = 0;
}

__global__ __launch_bounds__(kOccHistThreads) void occ_hist(const uint16_t* __restrict__ x,
                                                            uint32_t total, FastDiv cpr,
                                                            int64_t ld, uint32_t* __restrict__ ghist) {
    __shared__ uint32_t h[kOccBins];
    for (int i = threadIdx.x; i < kOccBins; i += kOccHistThreads) h[i] = 0;
    __syncthreads();
    for (uint32_t g = blockIdx.x * kOccHistThreads + threadIdx.x; g < total;
         g += gridDim.x * kOccHistThreads) {
        const uint32_t r = fastdiv(g, cpr);
        const uint32_t c = (g - r * cpr.d) * 8;
        const uint4 v = *(const uint4*)(x + (int64_t)r * ld + c);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            atomicAdd(&h[w[k] & 0x7FFFu], 1u);
            atomicAdd(&h[(w[k] >> 16) & 0x7FFFu], 1u);
        }
    }
    __syncthreads();
    for (int i = threadIdx.x; i < kOccBins; i += kOccHistThreads) {
        const uint32_t n = h[i];
        if (n) atomicAdd(&ghist[i], n);
    }
}

__device__ __forceinline__ uint64_t wave_incl_scan64(uint64_t v, int lane) {
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint64_t t = __shfl_up(v, d, 64);
        if (lane >= d) v += t;
    }
    return v;
}

// Exclusive prefix sum over a 1024-thread workgroup in thread order.
__device__ __forceinline__ uint64_t block_excl_scan64(uint64_t v, uint64_t* wtot) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint64_t inc = wave_incl_scan64(v, lane);
    if (lane == 63) wtot[wave] = inc;
    __syncthreads();
    uint64_t base = 0;
    for (int w = 0; w < wave; ++w) base += wtot[w];
    __syncthreads();
    return base + inc - v;
}

// The bin of the j-th smallest magnitude (1-based): the smallest b with
// count(bins <= b) >= j.  The histogram is copied with coalesced loads into
// LDS (one pad word per 32 bins, so thread t's 32 consecutive bins sit in
// distinct banks); thread t then owns bins [32 t, 32 t + 32).
__global__ __launch_bounds__(1024) void occ_select(const uint32_t* __restrict__ hist, uint64_t j,
                                                   uint32_t* __restrict__ params,
                                                   uint16_t* __restrict__ t_out) {
    __shared__ uint32_t h[kOccBins + kOccBins / 32];
    __shared__ uint64_t wtot[16];
    const int t = threadIdx.x;
#pragma unroll 8
    for (int i = t; i < kOccBins; i += 1024) h[i + (i >> 5)] = hist[i];
    __syncthreads();
    uint32_t c[32];
    uint64_t s = 0;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        c[i] = h[33 * t + i];
        s += c[i];
    }
    uint64_t before = block_excl_scan64(s, wtot);
    if (before < j && before + s >= j) {  // exactly one thread
        uint32_t b = 0;
        bool done = false;
#pragma unroll
        for (int i = 0; i < 32; ++i) {
            before += c[i];
            if (!done && before >= j) {
                b = 32 * t + i;
                done = true;
            }
        }
        params[0] = b;
        if (t_out) t_out[0] = (uint16_t)b;
    }
}

static constexpr int kOccUnroll = 4;  // chunks per clamp-quantise thread

template <int SR>
__device__ __forceinline__ void occ_chunk(uint4 v, uint32_t g, bool valid, FastDiv cpr, uint32_t tb,
                                          bool tfin,
                                          uint32_t k0, uint32_t k1, uint64_t off,
                                          uint8_t* __restrict__ codes, uint8_t* __restrict__ scales,
                                          uint8_t* __restrict__ mask,
                                          uint32_t* __restrict__ row_cnt) {
    const uint32_t r = fastdiv(g, cpr);
    const uint32_t c = (g - r * cpr.d) * 8;
    uint32_t w[4] = {v.x, v.y, v.z, v.w};
    uint32_t mb = 0;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        uint32_t lo = w[k] & 0xFFFFu, hi = w[k] >> 16;
        const bool olo = tfin && (lo & 0x7FFFu) > tb, ohi = tfin && (hi & 0x7FFFu) > tb;
        lo = olo ? ((lo & 0x8000u) | tb) : lo;
        hi = ohi ? ((hi & 0x8000u) | tb) : hi;
        w[k] = lo | (hi << 16);
        mb |= (olo ? 1u : 0u) << (2 * k);
        mb |= (ohi ? 1u : 0u) << (2 * k + 1);
    }
    if (!valid) mb = 0;
    if (valid) mask[g] = (uint8_t)mb;
    // the row's outlier count: one atomic per wave when the wave's valid
    // chunks lie in one row (the common case; lane 0 holds the wave's first
    // chunk, and if it is past the end so are all), else one per chunk
    // holding outliers.  Every lane of the wave runs this.
    const uint32_t n = (uint32_t)__builtin_popcount(mb);
    const uint32_t r_first = __builtin_amdgcn_readfirstlane(r);
    if (__builtin_amdgcn_ballot_w64(valid && r != r_first) == 0) {
        uint32_t sum = n;
#pragma unroll
        for (int m = 1; m < 64; m <<= 1) sum += (uint32_t)__shfl_xor((int)sum, m, 64);
        if (sum && __lane_id() == 0) atomicAdd(&row_cnt[r_first], sum);
    } else if (n) {
        atomicAdd(&row_cnt[r], n);
    }
    if (!valid) return;
    const uint32_t w0 = w[0], w1 = w[1], w2 = w[2], w3 = w[3];
    const u16x2_t m0 = __builtin_bit_cast(u16x2_t, w0 & 0x7FFF7FFFu);
    const u16x2_t m1 = __builtin_bit_cast(u16x2_t, w1 & 0x7FFF7FFFu);
    const u16x2_t m2 = __builtin_bit_cast(u16x2_t, w2 & 0x7FFF7FFFu);
    const u16x2_t m3 = __builtin_bit_cast(u16x2_t, w3 & 0x7FFF7FFFu);
    const u16x2_t mm = __builtin_elementwise_max(__builtin_elementwise_max(m0, m1),
                                                 __builtin_elementwise_max(m2, m3));
    const uint32_t amax = group_max_u32<4>(((uint32_t)max(mm.x, mm.y)) << 16);
    const bool nf = amax >= 0x7F800000u;
    const uint32_t byte = nf ? 0xFFu : e8m0_from_amax(amax);
    const float sc = e8m0_scale_f32(nf ? 0u : byte);
    uint32_t packed = 0;
    if (!SR) {
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w0), sc, 0);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w1), sc, 1);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w2), sc, 2);
        packed = __builtin_amdgcn_cvt_scalef32_pk_fp4_bf16(packed, __builtin_bit_cast(bf16x2_t, w3), sc, 3);
    } else {
        uint32_t wr[4];
        sr_words8((uint64_t)r * (uint64_t)(cpr.d * 8) + c + off, k0, k1, wr);
        const float xf[8] = {bf16_lo(w0), bf16_hi(w0), bf16_lo(w1), bf16_hi(w1),
                             bf16_lo(w2), bf16_hi(w2), bf16_lo(w3), bf16_hi(w3)};
        packed = sr_pack8(xf, sc, wr);
    }
    ((uint32_t*)codes)[g] = nf ? 0u : packed;
    if ((g & 3) == 0) scales[g >> 2] = (uint8_t)byte;
}

// A thread takes chunks g_u = (block * U + u) * 256 + tid, u < U: the four
// loads are issued before any arithmetic.  total % 4 == 0, so a quad's
// chunks are all in range or all out.
template <int SR>
__global__ __launch_bounds__(kOccThreads) void occ_clamp_quant(
    const uint16_t* __restrict__ x, uint32_t total, FastDiv cpr, int64_t ld,
    const uint32_t* __restrict__ params, uint32_t k0, uint32_t k1, uint64_t off,
    uint8_t* __restrict__ codes, uint8_t* __restrict__ scales, uint8_t* __restrict__ mask,
    uint32_t* __restrict__ row_cnt) {
    const uint32_t tb = params[0];
    const bool tfin = tb <= 0x7F80u;  // T itself not NaN
    uint4 v[kOccUnroll];
    uint32_t g[kOccUnroll];
#pragma unroll
    for (int u = 0; u < kOccUnroll; ++u) {
        g[u] = (blockIdx.x * kOccUnroll + u) * kOccThreads + threadIdx.x;
        v[u] = make_uint4(0u, 0u, 0u, 0u);
        if (g[u] < total) {
            const uint32_t r = fastdiv(g[u], cpr);
            v[u] = *(const uint4*)(x + (int64_t)r * ld + (g[u] - r * cpr.d) * 8);
        }
    }
#pragma unroll
    for (int u = 0; u < kOccUnroll; ++u)  // every lane: the row counts are summed across the wave
        occ_chunk<SR>(v[u], g[u], g[u] < total, cpr, tb, tfin, k0, k1, off, codes, scales, mask,
                      row_cnt);
}

// Thread t owns rows [t per, (t + 1) per); up to 16 rows per thread (16384
// rows) are held in registers, larger row counts re-read their counts.
__global__ __launch_bounds__(1024) void occ_scan(const uint32_t* __restrict__ row_cnt,
                                                 int64_t rows, int64_t* __restrict__ row_ptr) {
    __shared__ uint64_t wtot[16];
    const int64_t per = (rows + 1023) / 1024;
    const int64_t r0 = (int64_t)threadIdx.x * per;
    uint64_t s = 0;
    if (rows <= kOccScanLds) {
        // up to 8192 rows: counts and pointers staged in LDS, so that the
        // global loads and stores are coalesced (a thread's own run of
        // consecutive rows, read and written directly, puts one address per
        // lane 8 to 16 words apart into every instruction)
        __shared__ uint32_t cnt[kOccScanLds];
        __shared__ int64_t ptr[kOccScanLds];
        for (int64_t i = threadIdx.x; i < rows; i += 1024) cnt[i] = row_cnt[i];
        __syncthreads();
        uint32_t c[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            c[i] = (i < per && r0 + i < rows) ? cnt[r0 + i] : 0u;
            s += c[i];
        }
        uint64_t base = block_excl_scan64(s, wtot);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (i < per && r0 + i < rows) {
                ptr[r0 + i] = (int64_t)base;
                base += c[i];
            }
        }
        if (r0 < rows && r0 + per >= rows) row_ptr[rows] = (int64_t)base;  // the last owner
        __syncthreads();
        for (int64_t i = threadIdx.x; i < rows; i += 1024) row_ptr[i] = ptr[i];
        return;
    }
    if (per <= 16) {
        uint32_t c[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            c[i] = (i < per && r0 + i < rows) ? row_cnt[r0 + i] : 0u;
            s += c[i];
        }
        uint64_t base = block_excl_scan64(s, wtot);
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            if (i < per && r0 + i < rows) {
                row_ptr[r0 + i] = (int64_t)base;
                base += c[i];
            }
        }
        if (r0 < rows && r0 + per >= rows) row_ptr[rows] = (int64_t)base;  // the last owner
        return;
    }
    for (int64_t i = 0; i < per; ++i)
        if (r0 + i < rows) s += row_cnt[r0 + i];
    uint64_t base = block_excl_scan64(s, wtot);
    for (int64_t i = 0; i < per; ++i) {
        if (r0 + i < rows) {
            row_ptr[r0 + i] = (int64_t)base;
            base += row_cnt[r0 + i];
        }
    }
    if (r0 < rows && r0 + per >= rows) row_ptr[rows] = (int64_t)base;
}

__global__ __launch_bounds__(kOccThreads) void occ_fill(const uint16_t* __restrict__ x,
                                                        int64_t rows, int64_t cols, int64_t ld,
                                                        const uint8_t* __restrict__ mask,
                                                        const uint32_t* __restrict__ params,
                                                        const int64_t* __restrict__ row_ptr,
                                                        int32_t* __restrict__ col_idx,
                                                        float* __restrict__ vals) {
    const int lane = threadIdx.x & 63;
    const int64_t r = (int64_t)blockIdx.x * (kOccThreads / 64) + (threadIdx.x >> 6);
    if (r >= rows) return;  // uniform per wave
    const int64_t cpr = cols / 8;
    const uint32_t tb = params[0];
    int64_t base = row_ptr[r];
    const int64_t end = row_ptr[r + 1];
    if (base == end) return;
    const uint8_t* mrow = mask + r * cpr;
    const uint16_t* xrow = x + r * ld;
    for (int64_t b0 = 0; b0 < cpr; b0 += 64) {
        const int64_t bi = b0 + lane;
        uint32_t mb = bi < cpr ? mrow[bi] : 0u;
        const uint32_t cnt = __builtin_popcount(mb);
        const uint64_t inc = wave_incl_scan64(cnt, lane);
        int64_t pos = base + (int64_t)(inc - cnt);
        while (mb) {
            const int e = __builtin_ctz(mb);
            mb &= mb - 1;
            const int64_t col = bi * 8 + e;
            const uint32_t xv = xrow[col];
            const float xf = as_f32(xv << 16);
            const float cf = as_f32(((xv & 0x8000u) | tb) << 16);
            col_idx[pos] = (int32_t)col;
            vals[pos] = xf - cf;
            ++pos;
        }
        base += (int64_t)__shfl(inc, 63, 64);
    }
}

hipError_t launch_occ_quantize(const void* x, int64_t rows, int64_t cols, int64_t ld, uint64_t j,
                               bool sr, uint64_t seed, uint64_t off, uint8_t* codes,
                               uint8_t* scales, int64_t* row_ptr, int32_t* col_idx, float* vals,
                               uint16_t* t_out, void* ws, int n_cus, hipStream_t s) {
    const OccWs w = occ_ws(ws, rows);
    const uint16_t* xb = (const uint16_t*)x;
    const uint32_t total = (uint32_t)(rows * (cols / 8));
    const FastDiv cpr = make_fastdiv((uint32_t)(cols / 8));
    const uint32_t k0 = (uint32_t)seed, k1 = (uint32_t)(seed >> 32);
    const int64_t zn = rows > kOccBins ? rows : kOccBins;
    FP4Q_LAUNCH((occ_zero), dim3((unsigned)((zn + kOccThreads - 1) / kOccThreads)), kOccThreads, 0, s,
        w.hist, w.row_cnt, rows);
    const uint32_t hb = (total + kOccHistThreads - 1) / kOccHistThreads;
    FP4Q_LAUNCH((occ_hist), dim3(hb < (uint32_t)n_cus ? hb : (uint32_t)n_cus), kOccHistThreads, 0, s,
        xb, total, cpr, ld, w.hist);
    FP4Q_LAUNCH((occ_select), 1, 1024, 0, s, w.hist, j, w.params, t_out);
    const dim3 gq((total + kOccThreads * kOccUnroll - 1) / (kOccThreads * kOccUnroll));
    if (sr)
        FP4Q_LAUNCH((occ_clamp_quant<1>), gq, kOccThreads, 0, s, xb, total, cpr, ld, w.params, k0, k1, off,
                                                     codes, scales, w.mask, w.row_cnt);
    else
        FP4Q_LAUNCH((occ_clamp_quant<0>), gq, kOccThreads, 0, s, xb, total, cpr, ld, w.params, k0, k1, off,
                                                     codes, scales, w.mask, w.row_cnt);
    FP4Q_LAUNCH((occ_scan), 1, 1024, 0, s, w.row_cnt, rows, row_ptr);
    FP4Q_LAUNCH((occ_fill), dim3((unsigned)((rows + 3) / 4)), kOccThreads, 0, s,
        xb, rows, cols, ld, w.mask, w.params, row_ptr, col_idx, vals);
    return hipGetLastError();
}

__global__ __launch_bounds__(kOccThreads) void occ_spmm_kernel(
    int64_t N, const int64_t* __restrict__ row_ptr, const int32_t* __restrict__ col_idx,
    const float* __restrict__ vals, const uint16_t* __restrict__ w, int64_t ldw,
    float* __restrict__ y, int64_t ldy) {
    const int64_t r = blockIdx.x;
    const int64_t n0 = ((int64_t)blockIdx.y * kOccThreads + threadIdx.x) * 8;
    const int64_t e0 = row_ptr[r], e1 = row_ptr[r + 1];
    if (e0 == e1 || n0 >= N) return;
    float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
    // eight entries' weight rows are fetched before their products are
    // accumulated (in CSR order): the gathers overlap instead of chaining
    int64_t e = e0;
    for (; e + 8 <= e1; e += 8) {
        uint4 q[8];
        float v[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            q[u] = *(const uint4*)(w + (int64_t)col_idx[e + u] * ldw + n0);
            v[u] = vals[e + u];
        }
#pragma unroll
        for (int u = 0; u < 8; ++u) {
            const uint32_t qw[4] = {q[u].x, q[u].y, q[u].z, q[u].w};
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                acc[2 * i] = __builtin_fmaf(v[u], bf16_lo(qw[i]), acc[2 * i]);
                acc[2 * i + 1] = __builtin_fmaf(v[u], bf16_hi(qw[i]), acc[2 * i + 1]);
            }
        }
    }
    for (; e < e1; ++e) {
        const uint4 q = *(const uint4*)(w + (int64_t)col_idx[e] * ldw + n0);
        const float v = vals[e];
        const uint32_t qw[4] = {q.x, q.y, q.z, q.w};
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            acc[2 * i] = __builtin_fmaf(v, bf16_lo(qw[i]), acc[2 * i]);
            acc[2 * i + 1] = __builtin_fmaf(v, bf16_hi(qw[i]), acc[2 * i + 1]);
        }
    }
    float4* yp = (float4*)(y + r * ldy + n0);
    float4 a = yp[0], b = yp[1];
    a.x += acc[0];
    a.y += acc[1];
    a.z += acc[2];
    a.w += acc[3];
    b.x += acc[4];
    b.y += acc[5];
    b.z += acc[6];
    b.w += acc[7];
    yp[0] = a;
    yp[1] = b;
}

hipError_t launch_occ_spmm(int64_t M, int64_t N, const int64_t* row_ptr, const int32_t* col_idx,
                           const float* vals, const void* w, int64_t ldw, float* y, int64_t ldy,
                           hipStream_t s) {
    const dim3 grid((unsigned)M, (unsigned)((N / 8 + kOccThreads - 1) / kOccThreads));
    FP4Q_LAUNCH((occ_spmm_kernel), grid, kOccThreads, 0, s, N, row_ptr, col_idx, vals, (const uint16_t*)w,
                                                 ldw, y, ldy);
    return hipGetLastError();
}

}  // namespace fp4q
