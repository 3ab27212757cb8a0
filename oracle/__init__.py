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


def gemm_dense(a_codes, a_scales, b_codes, b_scales, block=32, rows=None, cols=None):
    """The same C = deq(A) deq(B)^T and S = sum |products| as gemm(), with
    the contraction done by a float64 matrix product of the exactly
    dequantised operands (a library primitive standing in for the sum; its
    rounding is K * 2^-53 * S at most, far below any tolerance used here).
    rows / cols: optional index arrays selecting rows of A / rows of B, so
    whole output rows or columns of a large product can be formed alone."""
    A = dequantize(a_codes if rows is None else _np.asarray(a_codes)[rows],
                   a_scales if rows is None else _np.asarray(a_scales)[rows], block)
    B = dequantize(b_codes if cols is None else _np.asarray(b_codes)[cols],
                   b_scales if cols is None else _np.asarray(b_scales)[cols], block)
    C = A @ B.T
    _np.abs(A, out=A)
    _np.abs(B, out=B)
    S = A @ B.T
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


def hcp_residual_dense(x, xq_codes, xq_scales, w, wq_codes, wq_scales, hot_idx, rows=None,
                       cols=None):
    """The residual of hcp_residual_entries for whole blocks of outputs:
    R = X_H W_H - Xq_H Wq_H over the hot channels H (float64 matrix products
    of the exact operand values), with S = |X_H| |W_H| + |Xq_H| |Wq_H|.
    x: bf16 bits [M, K]; w: bf16 bits [K, N]; wq K-major [N, K/2].
    rows / cols: optional index arrays of the outputs wanted."""
    hot = _np.asarray(hot_idx, _np.int64)
    xs = _c(x, _np.uint16) if rows is None else _np.asarray(x)[rows]
    ws = _c(w, _np.uint16) if cols is None else _np.asarray(w)[:, cols]
    xh = bf16_to_f64(_np.ascontiguousarray(xs[:, hot]))
    wh = bf16_to_f64(_np.ascontiguousarray(ws[hot, :]))
    xq = dequantize(xq_codes if rows is None else _np.asarray(xq_codes)[rows],
                    xq_scales if rows is None else _np.asarray(xq_scales)[rows], 32)[:, hot]
    wq = dequantize(wq_codes if cols is None else _np.asarray(wq_codes)[cols],
                    wq_scales if cols is None else _np.asarray(wq_scales)[cols], 32)[:, hot].T
    R = xh @ wh - xq @ wq
    S = _np.abs(xh) @ _np.abs(wh) + _np.abs(xq) @ _np.abs(wq)
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


def hcp_split_dense(x, w, hot_idx, rows=None, cols=None):
    """hcp_split_entries for whole blocks of outputs: X_H W_H over the hot
    channels (a float64 matrix product of the exact bf16 values) with the
    sum of |terms|.  x: bf16 bits [M, K]; w: bf16 bits [K, N]; rows / cols:
    optional index arrays of the outputs wanted."""
    hot = _np.asarray(hot_idx, _np.int64)
    xs = _np.asarray(x) if rows is None else _np.asarray(x)[rows]
    ws = _np.asarray(w) if cols is None else _np.asarray(w)[:, cols]
    xh = bf16_to_f64(_np.ascontiguousarray(xs[:, hot]))
    wh = bf16_to_f64(_np.ascontiguousarray(ws[hot, :]))
    return xh @ wh, _np.abs(xh) @ _np.abs(wh)


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
#
# The recipe of the outlier-dynamics page (sec. 4.1) transforms the backward
# pass's operands with a random Hadamard transform before quantising them.
# Read as the usual blockwise form: along the block axis every group of 32
# values x becomes y = 2^-2.5 * H32 * D * x, H32 the Sylvester
# (natural-order) Hadamard matrix with entries (-1)^popcount(i & j) and
# D = diag(+-1) from a sign mask, so that 2^-2.5 * H32 is orthogonal.  The
# oracle computes that definition in float64 (a matrix product, no
# evaluation order).  A device evaluates y in fp32; any evaluation as five
# levels of pairwise additions (a butterfly network, in any stride order),
# then a product by the rounded constant, lies within RHT_BOUND_ULPS fp32
# rounding units of 2^-2.5 * sum|x| of the exact value (each level adds at
# most one unit of the group's sum|x|; the constant and the product add two
# more), so
# the quantised result is checked for being one that some value within that
# bound gives (rht_check), and is exact wherever the bound crosses no
# rounding or scale boundary.

RHT_BOUND_ULPS = 8.0
_FLT_MAX = float(_np.finfo(_np.float32).max)


def hadamard32():
    """H32 of the definition: entry (i, j) = (-1)^popcount(i & j)."""
    i = _np.arange(32)
    pc = _np.array([bin(v).count("1") for v in range(32)])
    return _np.where(pc[i[:, None] & i[None, :]] % 2 == 1, -1.0, 1.0)


def _block_last(x, axis):
    """float64 view of x with the block axis last (COL: the transpose)."""
    x = _np.ascontiguousarray(x)
    v = bf16_to_f64(x) if x.dtype == _np.uint16 else x.astype(_np.float64)
    return _np.ascontiguousarray(v.T) if axis == COL else v


def _rht_groups(v, signs):
    """v float64 [R, n] (block axis last) -> exact y, the fp32 bound per
    element, and per group (R, n/32) the flags must_ff / may_ff: the group
    holds a non-finite input or its fp32 evaluation must overflow / may
    overflow."""
    R, n = v.shape
    if n % 32:
        raise ValueError("rht: the block axis must be a multiple of 32")
    d = _np.where(_np.asarray(signs, bool), -1.0, 1.0)
    g = (v * d[None, :]).reshape(R, n // 32, 32)
    fin = _np.isfinite(g).all(axis=2)
    gz = _np.where(fin[:, :, None], g, 0.0)
    s = gz @ hadamard32().T                 # H32 * D * x per group (H32 is symmetric)
    c = 2.0 ** -2.5
    sabs = _np.abs(gz).sum(axis=2)          # sum |x| per group
    u = 2.0 ** -24
    bound = RHT_BOUND_ULPS * u * c * sabs + 2.0 ** -149
    must_ff = ~fin | (_np.abs(s).max(axis=2) - 6 * u * sabs > 2.0 ** 128)
    may_ff = must_ff | (sabs * (1 + RHT_BOUND_ULPS * u) >= _FLT_MAX)
    y = (s * c).reshape(R, n)
    return y, _np.repeat(bound, 32, axis=1), must_ff, may_ff


def rht_exact(x, axis, signs):
    """The transform's definition y = 2^-2.5 * H32 * D * x per group of 32
    along the block axis, in float64.  x: bf16 bits or float32 [rows, cols];
    axis ROW = groups along columns, COL = along rows; signs: bool per
    position of the block axis (True = negate).  Returns (y float64 in x's
    orientation, bound float64: the largest distance of a correct fp32
    evaluation from y, element by element).  Groups holding a non-finite
    value give y = 0 there (see rht_check for how they are judged)."""
    y, b, _, _ = _rht_groups(_block_last(x, axis), signs)
    if axis == COL:
        return _np.ascontiguousarray(y.T), _np.ascontiguousarray(b.T)
    return y, b


def rht_quantize(x, axis, signs, round=RNE, seed=0, rng_offset=0):
    """A nominal quantisation of the transformed tensor: the exact transform
    rounded once to fp32 (one admissible evaluation), then the block-32
    quantiser (layouts, rounding and random counters as quantize); groups
    holding a non-finite input or overflowing fp32 get scale 0xFF."""
    v = _block_last(x, axis)
    y, _, must_ff, may_ff = _rht_groups(v, signs)
    with _np.errstate(over="ignore"):
        y32 = y.astype(_np.float32)
    ff = _np.repeat(must_ff, 32, axis=1)
    y32[ff] = _np.nan                       # the quantiser writes 0xFF for such groups
    src = _np.ascontiguousarray(y32.T) if axis == COL else y32
    return quantize(src, 32, axis, round, seed, rng_offset)


def _signed_val(codes):
    grid = _np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0])
    v = grid[codes & 7]
    return _np.where(codes & 8, -v, v)


def _unpack(codes):
    c = _np.ascontiguousarray(codes, _np.uint8)
    out = _np.empty((c.shape[0], 2 * c.shape[1]), _np.uint8)
    out[:, 0::2] = c & 0xF
    out[:, 1::2] = c >> 4
    return out


def _byte_of(a):
    """E8M0 byte of amax values a >= 0 given in float64: floor(log2 a) - 2
    clamped to [-127, 127], biased by 127; a = 0 gives 0."""
    a = _np.asarray(a, _np.float64)
    _, ex = _np.frexp(_np.where(a > 0, a, 1.0))
    e = _np.clip(ex - 1 - 2, -127, 127)
    return _np.where(a > 0, e + 127, 0).astype(_np.int64)


def rht_check(x, axis, signs, codes, scales, round=RNE, seed=0, rng_offset=0):
    """Is (codes, scales) the quantisation of some fp32 evaluation of the
    transform within the bound of the exact value?  For each group: the scale
    byte must be one that an amax within the bounds admits (0xFF only where
    the group holds a non-finite value or may overflow fp32; required where
    it must); under the byte given, each element's code must lie between the
    codes of y - bound and y + bound (nearest-even, or stochastic with the
    element's own random bits; both are monotone in y), a signed zero only
    where that sign is reachable.  Returns a dict with the counts of bad
    scale bytes and bad codes, the first bad position, and how many groups
    and elements were fixed uniquely by the bound (the exact ones) out of the
    groups and the elements of groups with a finite scale."""
    v = _block_last(x, axis)
    R, n = v.shape
    y, b, must_ff, may_ff = _rht_groups(v, signs)
    sc = _np.ascontiguousarray(scales, _np.uint8).astype(_np.int64)
    cd = _unpack(codes)
    if sc.shape != (R, n // 32) or cd.shape != (R, n):
        raise ValueError("rht_check: codes/scales do not have the quantised layout")
    ay = _np.abs(y).reshape(R, n // 32, 32)
    bb = b.reshape(R, n // 32, 32)
    blo = _byte_of(_np.maximum(ay - bb, 0.0).max(axis=2))
    bhi = _byte_of((ay + bb).max(axis=2))
    is_ff = sc == 0xFF
    ok_byte = _np.where(is_ff, may_ff, ~must_ff & (sc >= blo) & (sc <= bhi))
    # codes under the byte given (groups with 0xFF: all codes zero)
    e = _np.repeat(_np.where(is_ff, 127, sc) - 127, 32, axis=1)
    lo = _np.ldexp(y - b, -e)
    hi = _np.ldexp(y + b, -e)
    if round == RNE:
        c_lo, c_hi = rne_codes(lo), rne_codes(hi)
    else:
        u = sr_bits(seed, rng_offset, R * n).reshape((n, R) if axis == COL else (R, n))
        u = _np.ascontiguousarray(u.T) if axis == COL else u
        c_lo, c_hi = sr_codes(lo, u), sr_codes(hi, u)
    vg, vl, vh = _signed_val(cd), _signed_val(c_lo), _signed_val(c_hi)
    ok_code = (vg >= vl) & (vg <= vh)
    zero = (cd & 7) == 0
    ok_code &= ~zero | _np.where(cd & 8, (y - b) < 0, (y + b) > 0)
    ffe = _np.repeat(is_ff, 32, axis=1)
    ok_code = _np.where(ffe, cd == 0, ok_code)
    exact_groups = int(((blo == bhi) & ~may_ff).sum())
    exact_elems = int(((c_lo == c_hi) & ~ffe).sum())
    bad_s = _np.argwhere(~ok_byte)
    bad_c = _np.argwhere(~ok_code)
    first = None
    if bad_s.size:
        i, j = bad_s[0]
        first = ("scale", (int(i), int(j)), int(sc[i, j]), (int(blo[i, j]), int(bhi[i, j])))
    elif bad_c.size:
        i, j = bad_c[0]
        first = ("code", (int(i), int(j)), int(cd[i, j]), (int(c_lo[i, j]), int(c_hi[i, j])))
    return {"bad_scales": int(bad_s.shape[0]), "bad_codes": int(bad_c.shape[0]),
            "exact_groups": exact_groups, "groups": int(sc.size),
            "exact_elems": exact_elems, "elems": int((~ffe).sum()), "first_bad": first}


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
