"""numpy front end of the plain CPU oracle (oracle/fp4q_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it; the product library never does.
It shares no code with the HIP path.  bf16 tensors travel as numpy ``uint16``
bit patterns, fp32 as ``float32``; every result the C side computes in double
is returned as ``float64`` and rounded to an output dtype only by
:func:`round_f32` / :func:`round_bf16`.
"""
import ctypes as _ct
import os as _os

import numpy as _np

from . import build as _build

F32, BF16 = 0, 1
ROW, COL = 0, 1
RNE, SR = 0, 1
STE, DGE = 0, 1

_lib = None


def lib():
    """Load oracle/liboracle.so, compiling it first only if it is missing."""
    global _lib
    if _lib is None:
        if not _os.path.exists(_build.LIB):
            _build.build()
        L = _ct.CDLL(_build.LIB)
        P, I64, I32, U64, D = _ct.c_void_p, _ct.c_int64, _ct.c_int, _ct.c_uint64, _ct.c_double
        sig = {
            "orc_e2m1_value": (D, [I32]),
            "orc_e8m0_byte": (I32, [_ct.c_uint32]),
            "orc_rne_code": (I32, [D]),
            "orc_sr_code": (I32, [D, _ct.c_uint32]),
            "orc_philox4x32": (None, [P, P, I32, P]),
            "orc_sr_bits": (_ct.c_uint32, [U64, U64]),
            "orc_quantize": (I32, [P, I32, I64, I64, I64, I32, I32, I32, U64, U64, P, P]),
            "orc_dequantize": (None, [P, P, I64, I64, I32, P]),
            "orc_quantize_2d": (I32, [P, I32, I64, I64, I64, I32, I32, U64, U64, P, P, P, P]),
            "orc_round_f32": (None, [P, P, I64]),
            "orc_round_bf16": (None, [P, P, I64]),
            "orc_bf16_from_double": (_ct.c_uint16, [D]),
            "orc_dge_f": (D, [D, D, D]),
            "orc_dge_fprime": (D, [D, D, D, D]),
            "orc_grad_estimate": (I32, [I32, P, I32, P, I32, I64, I64, I32, I32, D, D, P, P]),
            "orc_gemm": (None, [I64, I64, I64, P, P, P, P, I32, P, P]),
            "orc_gemm_entries": (None, [I64, P, P, P, P, I32, I64, P, P, P, P]),
            "orc_gemm_intblock": (None, [I64, I64, I64, P, P, P, P, I32, P]),
            "orc_hcp_residual_entries": (None, [I64, I64, P, P, P, P, P, P, P, I32, I64, P, P,
                                                P, P]),
            "orc_e8m0_bytes": (None, [P, I64, P]),
            "orc_rne_codes": (None, [P, I64, P]),
            "orc_sr_codes": (None, [P, P, I64, P]),
            "orc_sr_bits_range": (None, [U64, U64, I64, P]),
            "orc_dge_f_many": (None, [P, P, I64, D, P]),
            "orc_dge_fprime_many": (None, [P, P, I64, D, D, P]),
        }
        for name, (res, args) in sig.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def _p(a):
    return a.ctypes.data_as(_ct.c_void_p)


def _c(a, dtype):
    return _np.ascontiguousarray(a, dtype=dtype)


def _dtype_of(x):
    if x.dtype == _np.uint16:
        return BF16
    if x.dtype == _np.float32:
        return F32
    raise TypeError("oracle takes float32 arrays or bf16 as uint16 bit patterns")


# --- element level ---------------------------------------------------------

def e2m1_value(code):
    return lib().orc_e2m1_value(int(code))


def e8m0_byte(amax_bits):
    return lib().orc_e8m0_byte(int(amax_bits) & 0x7FFFFFFF)


def e8m0_bytes(bits):
    bits = _c(bits, _np.uint32)
    out = _np.empty(bits.shape, _np.uint8)
    lib().orc_e8m0_bytes(_p(bits), bits.size, _p(out))
    return out


def rne_codes(y):
    y = _c(y, _np.float64)
    out = _np.empty(y.shape, _np.uint8)
    lib().orc_rne_codes(_p(y), y.size, _p(out))
    return out


def sr_codes(y, u16):
    y = _c(y, _np.float64)
    u = _c(u16, _np.uint32)
    out = _np.empty(y.shape, _np.uint8)
    lib().orc_sr_codes(_p(y), _p(u), y.size, _p(out))
    return out


def philox4x32(ctr, key, rounds=10):
    c = _c(ctr, _np.uint32)
    k = _c(key, _np.uint32)
    out = _np.empty(4, _np.uint32)
    lib().orc_philox4x32(_p(c), _p(k), int(rounds), _p(out))
    return out


def sr_bits(seed, pos0, n):
    out = _np.empty(int(n), _np.uint32)
    lib().orc_sr_bits_range(int(seed), int(pos0), int(n), _p(out))
    return out


def dge_f(t, delta, k):
    t = _c(t, _np.float64)
    d = _c(_np.broadcast_to(delta, t.shape), _np.float64)
    out = _np.empty(t.shape, _np.float64)
    lib().orc_dge_f_many(_p(t), _p(d), t.size, float(k), _p(out))
    return out


def dge_fprime(t, delta, k, clamp_max):
    t = _c(t, _np.float64)
    d = _c(_np.broadcast_to(delta, t.shape), _np.float64)
    out = _np.empty(t.shape, _np.float64)
    lib().orc_dge_fprime_many(_p(t), _p(d), t.size, float(k), float(clamp_max), _p(out))
    return out


# --- tensor level ----------------------------------------------------------

def quantize(x, block, axis=ROW, round=RNE, seed=0, rng_offset=0):
    """x: [rows, cols] float32 or bf16-as-uint16.  Returns (codes, scales):
    ROW -> [rows, cols/2], [rows, cols/block]; COL -> [cols, rows/2], [cols, rows/block]."""
    x = _np.ascontiguousarray(x)
    dt = _dtype_of(x)
    rows, cols = x.shape
    if axis == ROW:
        codes = _np.empty((rows, cols // 2), _np.uint8)
        scales = _np.empty((rows, cols // block), _np.uint8)
    else:
        codes = _np.empty((cols, rows // 2), _np.uint8)
        scales = _np.empty((cols, rows // block), _np.uint8)
    rc = lib().orc_quantize(_p(x), dt, rows, cols, cols, int(block), int(axis), int(round),
                            int(seed), int(rng_offset), _p(codes), _p(scales))
    if rc != 0:
        raise ValueError("oracle quantize: unsupported shape/block")
    return codes, scales


def quantize_2d(x, tile=32, round=RNE, seed=0, rng_offset=0):
    """Two-dimensional block scaling (outlier-dynamics page, sec. 4.1): one
    scale per tile x tile square.  x: [rows, cols] float32 or bf16-as-uint16.
    Returns (codes_r [rows, cols/2], scales_r [rows, cols/tile],
             codes_c [cols, rows/2], scales_c [cols, rows/tile]): the same
    quantised values in the ROW and the COL (K-major) layout."""
    x = _np.ascontiguousarray(x)
    dt = _dtype_of(x)
    rows, cols = x.shape
    cr = _np.empty((rows, cols // 2), _np.uint8)
    sr = _np.empty((rows, cols // tile), _np.uint8)
    cc = _np.empty((cols, rows // 2), _np.uint8)
    sc = _np.empty((cols, rows // tile), _np.uint8)
    rc = lib().orc_quantize_2d(_p(x), dt, rows, cols, cols, int(tile), int(round), int(seed),
                               int(rng_offset), _p(cr), _p(sr), _p(cc), _p(sc))
    if rc != 0:
        raise ValueError("oracle quantize_2d: unsupported shape/tile")
    return cr, sr, cc, sc


def dequantize(codes, scales, block):
    """codes [rows, k/2], scales [rows, k/block] -> float64 [rows, k] (exact)."""
    codes = _c(codes, _np.uint8)
    scales = _c(scales, _np.uint8)
    rows, half = codes.shape
    k = 2 * half
    out = _np.empty((rows, k), _np.float64)
    lib().orc_dequantize(_p(codes), _p(scales), rows, k, int(block), _p(out))
    return out


def round_f32(v):
    v = _c(v, _np.float64)
    out = _np.empty(v.shape, _np.float32)
    lib().orc_round_f32(_p(v), _p(out), v.size)
    return out


def round_bf16(v):
    """Round-to-nearest-even of float64 straight to bf16; returns uint16 bits."""
    v = _c(v, _np.float64)
    out = _np.empty(v.shape, _np.uint16)
    lib().orc_round_bf16(_p(v), _p(out), v.size)
    return out


def bf16_to_f64(bits):
    """Exact widening of bf16 bit patterns to float64."""
    b = _c(bits, _np.uint16).astype(_np.uint32) << 16
    return b.view(_np.float32).astype(_np.float64)


def grad_estimate(mode, x, g, block=32, axis=ROW, k=5.0, clamp_max=3.0):
    """Returns (d, out) in float64: the derivative factor and g*d, both exact
    before the final rounding to an output dtype."""
    g = _np.ascontiguousarray(g)
    rows, cols = g.shape
    if x is None:
        x = _np.zeros((1, 1), _np.float32)
    x = _np.ascontiguousarray(x)
    d = _np.empty((rows, cols), _np.float64)
    out = _np.empty((rows, cols), _np.float64)
    rc = lib().orc_grad_estimate(int(mode), _p(x), _dtype_of(x), _p(g), _dtype_of(g), rows,
                                 cols, int(block), int(axis), float(k), float(clamp_max),
                                 _p(d), _p(out))
    if rc != 0:
        raise ValueError("oracle grad_estimate: unsupported shape/block")
    return d, out


def gemm(a_codes, a_scales, b_codes, b_scales, block=32):
    """C = deq(A) deq(B)^T in double, plus S = sum |products|."""
    ac, as_, bc, bs = (_c(t, _np.uint8) for t in (a_codes, a_scales, b_codes, b_scales))
    M, N, K = ac.shape[0], bc.shape[0], 2 * ac.shape[1]
    C = _np.empty((M, N), _np.float64)
    S = _np.empty((M, N), _np.float64)
    lib().orc_gemm(M, N, K, _p(ac), _p(as_), _p(bc), _p(bs), int(block), _p(C), _p(S))
    return C, S


def gemm_intblock(a_codes, a_scales, b_codes, b_scales, block=32):
    ac, as_, bc, bs = (_c(t, _np.uint8) for t in (a_codes, a_scales, b_codes, b_scales))
    M, N, K = ac.shape[0], bc.shape[0], 2 * ac.shape[1]
    C = _np.empty((M, N), _np.float64)
    lib().orc_gemm_intblock(M, N, K, _p(ac), _p(as_), _p(bc), _p(bs), int(block), _p(C))
    return C


def gemm_entries(a_codes, a_scales, b_codes, b_scales, ii, jj, block=32):
    ac, as_, bc, bs = (_c(t, _np.uint8) for t in (a_codes, a_scales, b_codes, b_scales))
    K = 2 * ac.shape[1]
    ii = _c(ii, _np.int64)
    jj = _c(jj, _np.int64)
    C = _np.empty(ii.shape, _np.float64)
    S = _np.empty(ii.shape, _np.float64)
    lib().orc_gemm_entries(K, _p(ac), _p(as_), _p(bc), _p(bs), int(block), ii.size, _p(ii),
                           _p(jj), _p(C), _p(S))
    return C, S


def hcp_residual_entries(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx, ii, jj):
    """Residual sum_{c in H} X[i,c]W[c,j] - Xq[i,c]Wq[c,j] at sampled (ii, jj).
    x: bf16 bits [M, K]; w: bf16 bits [K, N]; wq K-major [N, K/2]."""
    x = _c(x, _np.uint16)
    w = _c(w, _np.uint16)
    K, N = w.shape
    xqc, xqs, wqc, wqs = (_c(t, _np.uint8) for t in (xq_codes, xq_scales, wq_codes, wq_scales))
    hot = _c(hot_idx, _np.int32)
    ii = _c(ii, _np.int64)
    jj = _c(jj, _np.int64)
    R = _np.empty(ii.shape, _np.float64)
    S = _np.empty(ii.shape, _np.float64)
    lib().orc_hcp_residual_entries(N, K, _p(x), _p(xqc), _p(xqs), _p(w), _p(wqc), _p(wqs),
                                   _p(hot), hot.size, ii.size, _p(ii), _p(jj), _p(R), _p(S))
    return R, S


def hcp_split_entries(x, w, hot_idx, ii, jj):
    """The split reading of the hot-channel compensation (outlier-dynamics
    page, sec. 3.1-3.2): the hot channels' own bf16 product
    sum_{c in H} X[i,c] W[c,j] at sampled (ii, jj), added to the product of the
    operands quantised with H zeroed.  float64 (every bf16 x bf16 product is
    exact; |H| terms), with the sum of |terms|.
    x: bf16 bits [M, K]; w: bf16 bits [K, N]."""
    xd = bf16_to_f64(_c(x, _np.uint16))
    wd = bf16_to_f64(_c(w, _np.uint16))
    hot = _c(hot_idx, _np.int64)
    ii = _c(ii, _np.int64)
    jj = _c(jj, _np.int64)
    R = _np.zeros(ii.shape, _np.float64)
    S = _np.zeros(ii.shape, _np.float64)
    for c in hot:  # one hot channel at a time, in the list's order
        t = xd[ii, c] * wd[c, jj]
        R += t
        S += _np.abs(t)
    return R, S


def channel_quant_error(x, block=32):
    """Per-channel (per-column) quantisation error of X under the ROW
    nearest-even MXFP4 quantisation: e_c = sum_i (x_ic - deq(Q(x))_ic)^2, in
    float64 (the ranking quantity of the hot-channel choice, outlier-dynamics
    page, sec. 4.1).  A block with a non-finite element dequantises to NaN, so
    its channels' errors are NaN.  x: bf16 bits or float32 [rows, cols]."""
    x = _np.ascontiguousarray(x)
    codes, scales = quantize(x, block, ROW, RNE)
    xd = bf16_to_f64(x) if x.dtype == _np.uint16 else x.astype(_np.float64)
    d = xd - dequantize(codes, scales, block)
    return (d * d).sum(axis=0)


def hot_channels(x, n_hot, block=32):
    """The n_hot channels of largest quantisation error (outlier-dynamics
    page, sec. 4.1: the top 9% of channels by error are kept in high
    precision), returned in ascending index order as int32.  Ranking: larger
    error first, NaN above every number, equal errors to the lower index."""
    e = channel_quant_error(x, block)
    idx = _np.arange(e.size)
    nan = _np.isnan(e)
    order = _np.lexsort((idx, -_np.where(nan, 0.0, e), ~nan))
    return _np.sort(order[:int(n_hot)]).astype(_np.int32), e


# --- random Hadamard transform before quantisation ------------------------

RHT_C = _np.float32(2.0 ** -2.5)   # 1/sqrt(32) rounded to fp32


def rht_transform(x, axis, signs):
    """The blockwise random Hadamard transform the recipe of the
    outlier-dynamics page (sec. 4.1) applies before backward quantisation,
    along the block axis in groups of 32: y = c * H32 * D * x per group, with
    D = diag(+-1) from `signs` (bool per position along the axis, True =
    negate), H32 the Sylvester (natural-order) Hadamard matrix, entries
    (-1)^popcount(i & j), and c = fl32(2^-2.5), so c*H32 is orthogonal up to
    rounding.  Evaluated in fp32, the precision the codes are decided in: the
    butterflies (a, b) -> (a + b, a - b) on pairs (i, i + s), bit s of i
    clear, for s = 1, 2, 4, 8, 16 in that order, then the product by c.
    x: bf16 bits or float32 [rows, cols]; axis ROW = along columns,
    COL = along rows.  Returns float32 [rows, cols]."""
    x = _np.ascontiguousarray(x)
    v = bf16_to_f64(x).astype(_np.float32) if x.dtype == _np.uint16 else x.astype(_np.float32)
    if axis == COL:
        v = _np.ascontiguousarray(v.T)
    rows, n = v.shape
    if n % 32:
        raise ValueError("rht_transform: the block axis must be a multiple of 32")
    sg = _np.asarray(signs, bool)
    v = _np.where(sg[None, :], -v, v).astype(_np.float32)
    v = v.reshape(rows, n // 32, 32)
    s = 1
    with _np.errstate(over="ignore", invalid="ignore"):  # fp32 overflow -> Inf/NaN, as defined
        while s < 32:
            w = v.reshape(rows, n // 32, 32 // (2 * s), 2, s)
            a = w[:, :, :, 0, :]
            b = w[:, :, :, 1, :]
            v = _np.stack([a + b, a - b], axis=3).reshape(rows, n // 32, 32)
            s *= 2
        v = (v * RHT_C).astype(_np.float32).reshape(rows, n)
    return _np.ascontiguousarray(v.T) if axis == COL else v


def rht_quantize(x, axis, signs, round=RNE, seed=0, rng_offset=0):
    """Block-32 quantisation of the transformed tensor: rht_transform(x) fed
    to the quantiser (layouts, rounding and random counters as quantize)."""
    y = rht_transform(x, axis, signs)
    return quantize(y, 32, axis, round, seed, rng_offset)


# --- outlier clamping and compensation (OCC) -------------------------------

def occ_threshold(x, quantile=0.99):
    """The clamp threshold of the outlier clamping and compensation on the
    MSRA FP4-training summary page (sec. 三): the `quantile` quantile of |x|
    over the whole tensor, as the order statistic T = a_j of the ascending
    magnitudes a_1 <= ... <= a_n with j = ceil(quantile * n) (NaN ranks above
    every number).  Returns (T as float64, nnz = #{|x| > T})."""
    xd = bf16_to_f64(x) if _np.asarray(x).dtype == _np.uint16 else _np.asarray(x, _np.float64)
    a = _np.sort(_np.abs(xd).reshape(-1))            # NaN sorts last
    n = a.size
    j = min(max(int(_np.ceil(quantile * n)), 1), n)
    t = a[j - 1]
    return t, int(_occ_outliers(xd, t).sum())


def _occ_outliers(xd, t):
    """|x| ranks above T, NaN ranking above every number (so with a finite T
    the NaN elements are outliers; with a NaN T there are none)."""
    if _np.isnan(t):
        return _np.zeros(xd.shape, bool)
    return (_np.abs(xd) > t) | _np.isnan(xd)


def occ_split(x, t):
    """Clamp and residual (same page, sec. 三 and 六): the outliers (|x| > T,
    and NaN while T is finite) become sign(x) T (exact in bf16: T is one of x's magnitudes); the
    residual R = x - clamp(x), nonzero only there, as CSR with columns
    ascending in each row and fp32 values (the exact difference rounded once
    to fp32).  x: bf16 bits [rows, cols].  Returns (clamped bf16 bits,
    row_ptr int64 [rows + 1], col_idx int32, vals float32)."""
    x = _c(x, _np.uint16)
    xd = bf16_to_f64(x)
    out = _occ_outliers(xd, t)
    tb = _np.uint16(_np.float32(t).view(_np.uint32) >> 16)
    clamped = _np.where(out, (x & _np.uint16(0x8000)) | tb, x).astype(_np.uint16)
    resid = xd - bf16_to_f64(clamped)
    rows, cols = x.shape
    r_idx, c_idx = _np.nonzero(out)                  # row-major order: rows, then columns
    row_ptr = _np.zeros(rows + 1, _np.int64)
    _np.add.at(row_ptr, r_idx + 1, 1)
    row_ptr = _np.cumsum(row_ptr)
    vals = round_f32(resid[r_idx, c_idx])
    return clamped, row_ptr, c_idx.astype(_np.int32), vals


def occ_spmm(row_ptr, col_idx, vals, w):
    """The sparse compensation product R W (float64, exact products; the
    sum of |terms| alongside): R from occ_split [rows, K], w bf16 bits [K, N]."""
    wd = bf16_to_f64(_c(w, _np.uint16))
    rows = row_ptr.size - 1
    out = _np.zeros((rows, wd.shape[1]), _np.float64)
    mag = _np.zeros_like(out)
    for i in range(rows):
        for e in range(int(row_ptr[i]), int(row_ptr[i + 1])):
            t = float(vals[e]) * wd[int(col_idx[e])]
            out[i] += t
            mag[i] += _np.abs(t)
    return out, mag
