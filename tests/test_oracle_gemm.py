"""Pins of the oracle's FP4 GEMM and hot-channel residual: two formulations
(double sums of dequantised values / exact integer block sums), a library
matmul of the dequantised operands, identity-coded operands, exhaustive 1x1x32
code pairs across scale bytes, the error-bound quantity S, and the residual's
special cases (empty hot set, all channels hot, operands already on the grid)."""
import numpy as np
import pytest

from mxfp4_block_scaled_fp4q_amd import inputs


def _e2m1(code):
    s = -1.0 if code & 8 else 1.0
    e = (code >> 1) & 3
    m = code & 1
    return s * (0.5 * m if e == 0 else 2.0 ** (e - 1) * (1 + 0.5 * m))


def _qpair(orc, shape_a, shape_b, seed):
    a = inputs.with_outliers(inputs.normal(shape_a, seed), seed + 1, 20, 50.0)
    b = inputs.with_outliers(inputs.normal(shape_b, seed + 2), seed + 3, 20, 50.0)
    return orc.quantize(a, 32), orc.quantize(b, 32)


def test_gemm_formulations_and_matmul(orc):
    (ac, as_), (bc, bs) = _qpair(orc, (48, 128), (40, 128), 21)
    C, S = orc.gemm(ac, as_, bc, bs)
    Ci = orc.gemm_intblock(ac, as_, bc, bs)
    assert np.all(np.abs(C - Ci) <= 1e-13 * S)
    A = orc.dequantize(ac, as_, 32)
    B = orc.dequantize(bc, bs, 32)
    Cm = A @ B.T
    assert np.all(np.abs(C - Cm) <= 1e-13 * S)
    assert np.allclose(S, np.abs(A) @ np.abs(B).T, rtol=1e-13, atol=0)
    assert np.all(S >= np.abs(C))
    # entry-wise sampler agrees with the full product
    ii = np.array([0, 47, 13, 5])
    jj = np.array([0, 39, 7, 33])
    Ce, Se = orc.gemm_entries(ac, as_, bc, bs, ii, jj)
    assert np.array_equal(Ce, C[ii, jj]) and np.array_equal(Se, S[ii, jj])


def test_gemm_identity_coded(orc):
    """B codes 1.0 on the diagonal (byte 127): C = deq(A) exactly."""
    (ac, as_), _ = _qpair(orc, (32, 64), (1, 64), 31)
    K = 64
    bc = np.zeros((K, K // 2), np.uint8)
    for j in range(K):
        bc[j, j // 2] = (2 << 4) if j & 1 else 2
    bs = np.full((K, K // 32), 127, np.uint8)
    C, _ = orc.gemm(ac, as_, bc, bs)
    assert np.array_equal(C, orc.dequantize(ac, as_, 32))


def test_gemm_zero_and_single_block(orc):
    ac = np.zeros((4, 64), np.uint8)
    as_ = np.full((4, 4), 127, np.uint8)
    bc = np.zeros((3, 64), np.uint8)
    bs = np.full((3, 4), 100, np.uint8)
    C, S = orc.gemm(ac, as_, bc, bs)
    assert np.all(C == 0) and np.all(S == 0)
    ac[1, 16:32] = 0x77  # block 1 of row 1: all 6.0
    bc[2, 16:32] = 0xAA  # block 1 of row 2: all -1.0
    as_[1, 1] = 130
    bs[2, 1] = 120
    C, _ = orc.gemm(ac, as_, bc, bs)
    want = 32 * 6.0 * -1.0 * 2.0 ** (130 - 127) * 2.0 ** (120 - 127)
    assert C[1, 2] == want
    C[1, 2] = 0
    assert np.all(C == 0)


def test_gemm_1x1x32_exhaustive_code_pairs(orc):
    """Every pair of codes, in every lane position, across a sweep of scale
    bytes: C = 32 * v(ca) v(cb) 2^(ea + eb - 254) for a block of equal codes,
    and lane-wise for a mixed block."""
    for ea, eb in [(127, 127), (0, 254), (1, 1), (200, 60), (127, 0), (254, 254)]:
        for ca in range(16):
            ac = np.full((1, 16), ca | (ca << 4), np.uint8)
            as_ = np.array([[ea]], np.uint8)
            bcs = np.array([[cb | (cb << 4)] * 16 for cb in range(16)], np.uint8)
            bss = np.full((16, 1), eb, np.uint8)
            C, _ = orc.gemm(ac, as_, bcs, bss)
            Ci = orc.gemm_intblock(ac, as_, bcs, bss)
            want = np.array([32 * _e2m1(ca) * _e2m1(cb) * 2.0 ** (ea + eb - 254)
                             for cb in range(16)])
            assert np.array_equal(C[0], want) and np.array_equal(Ci[0], want)
    rng = np.random.default_rng(2)
    a = rng.integers(0, 16, 32)
    b = rng.integers(0, 16, 32)
    ac = (a[0::2] | (a[1::2] << 4)).astype(np.uint8)[None]
    bc = (b[0::2] | (b[1::2] << 4)).astype(np.uint8)[None]
    C, _ = orc.gemm(ac, np.array([[127]], np.uint8), bc, np.array([[127]], np.uint8))
    assert C[0, 0] == sum(_e2m1(int(p)) * _e2m1(int(q)) for p, q in zip(a, b))


def test_gemm_nan_scale(orc):
    ac = np.full((1, 32), 0x22, np.uint8)
    as_ = np.array([[0xFF, 127]], np.uint8)
    bc = np.full((1, 32), 0x22, np.uint8)
    bs = np.array([[127, 127]], np.uint8)
    assert np.isnan(orc.gemm(ac, as_, bc, bs)[0][0, 0])
    assert np.isnan(orc.gemm_intblock(ac, as_, bc, bs)[0, 0])


def _hcp_case(orc, M, K, N, seed):
    x = inputs.to_bf16_bits(inputs.normal((M, K), seed))
    w = inputs.to_bf16_bits(inputs.normal((K, N), seed + 1, 0.02))
    xqc, xqs = orc.quantize(x, 32)
    wqc, wqs = orc.quantize(w, 32, axis=orc.COL)
    return x, w, xqc, xqs, wqc, wqs


def test_hcp_empty_and_full(orc):
    M, K, N = 16, 64, 24
    x, w, xqc, xqs, wqc, wqs = _hcp_case(orc, M, K, N, 41)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ii, jj = ii.ravel(), jj.ravel()
    R, S = orc.hcp_residual_entries(x, xqc, xqs, w, wqc, wqs, np.zeros(0, np.int32), ii, jj)
    assert np.all(R == 0) and np.all(S == 0)
    # every channel hot: base + residual = the plain product of the bf16 inputs
    C, Sb = orc.gemm(xqc, xqs, wqc, wqs)
    R, S = orc.hcp_residual_entries(x, xqc, xqs, w, wqc, wqs, np.arange(K, dtype=np.int32),
                                    ii, jj)
    Y = C.ravel() + R
    Xd = orc.bf16_to_f64(x)
    Wd = orc.bf16_to_f64(w)
    want = (Xd @ Wd).ravel()
    assert np.all(np.abs(Y - want) <= 1e-12 * (Sb.ravel() + S))


def test_hcp_on_grid_is_zero_and_linear(orc):
    M, K, N = 8, 64, 16
    # X and W whose hot columns/rows are already FP4 values times the block
    # scale: quantisation is exact there, so the residual vanishes
    rng = np.random.default_rng(9)
    grid = np.array([0, 0.5, 1, 1.5, 2, 3, 4, 6.0])
    xf = (grid[rng.integers(0, 8, (M, K))] * rng.choice([-1, 1], (M, K))).astype(np.float32)
    xf[:, 0] = 4.0
    xf[:, 32] = 6.0
    wf = (grid[rng.integers(0, 8, (K, N))] * 0.25).astype(np.float32)
    wf[0, :] = 1.0
    wf[32, :] = 1.5
    x = inputs.to_bf16_bits(xf)
    w = inputs.to_bf16_bits(wf)
    xqc, xqs = orc.quantize(x, 32)
    wqc, wqs = orc.quantize(w, 32, axis=orc.COL)
    hot = np.array([1, 5, 33, 63], np.int32)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    R, _ = orc.hcp_residual_entries(x, xqc, xqs, w, wqc, wqs, hot, ii.ravel(), jj.ravel())
    assert np.all(R == 0)
    # residual is additive over disjoint hot sets
    x, w, xqc, xqs, wqc, wqs = _hcp_case(orc, M, K, N, 51)
    h1 = np.array([2, 9, 40], np.int32)
    h2 = np.array([11, 50], np.int32)
    Ra, _ = orc.hcp_residual_entries(x, xqc, xqs, w, wqc, wqs, h1, ii.ravel(), jj.ravel())
    Rb, _ = orc.hcp_residual_entries(x, xqc, xqs, w, wqc, wqs, h2, ii.ravel(), jj.ravel())
    Rab, S = orc.hcp_residual_entries(x, xqc, xqs, w, wqc, wqs, np.concatenate([h1, h2]),
                                      ii.ravel(), jj.ravel())
    assert np.all(np.abs(Ra + Rb - Rab) <= 1e-14 * S)


def test_hcp_split_brute_force_and_identities(orc):
    """Split reading: the residual equals a plain triple loop on a tiny case;
    no hot channels gives zero; with every channel hot the quantised operands
    are all zero and the residual alone is the exact bf16 product."""
    M, K, N = 3, 64, 5
    x, w, _, _, _, _ = _hcp_case(orc, M, K, N, 61)
    hot = np.array([1, 5, 33, 62], np.int32)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ii, jj = ii.ravel(), jj.ravel()
    R, S = orc.hcp_split_entries(x, w, hot, ii, jj)
    xd, wd = orc.bf16_to_f64(x), orc.bf16_to_f64(w)
    for n, (i, j) in enumerate(zip(ii, jj)):
        acc = 0.0
        for c in hot:
            acc += xd[i, c] * wd[c, j]
        assert R[n] == acc
    R0, S0 = orc.hcp_split_entries(x, w, np.zeros(0, np.int32), ii, jj)
    assert np.all(R0 == 0) and np.all(S0 == 0)
    allh = np.arange(K, dtype=np.int32)
    xz, wz = x.copy(), w.copy()
    xz[:, allh] = 0
    wz[allh, :] = 0
    xqc, xqs = orc.quantize(xz, 32)
    wqc, wqs = orc.quantize(wz, 32, axis=orc.COL)
    C, _ = orc.gemm(xqc, xqs, wqc, wqs)
    assert np.all(C == 0)
    R, S = orc.hcp_split_entries(x, w, allh, ii, jj)
    assert np.all(np.abs(C.ravel() + R - (xd @ wd).ravel()) <= 1e-12 * S)


def test_gemm_dense_equals_loop_form(orc):
    """gemm_dense (matrix product of the dequantised operands, with row and
    column selections) against the plain loop and the integer-block sum,
    including a NaN scale and ragged sizes."""
    (ac, as_), (bc, bs) = _qpair(orc, (37, 192), (29, 192), 23)
    as_ = as_.copy()
    as_[3, 2] = 0xFF
    C, S = orc.gemm(ac, as_, bc, bs)
    Cd, Sd = orc.gemm_dense(ac, as_, bc, bs)
    nan = np.isnan(C)
    assert np.array_equal(nan, np.isnan(Cd)) and nan[3].all() and nan.sum() == 29
    ok = ~nan
    assert np.all(np.abs(C[ok] - Cd[ok]) <= 1e-13 * S[ok])
    assert np.allclose(S[ok], Sd[ok], rtol=1e-13, atol=0)
    Ci = orc.gemm_intblock(ac, as_, bc, bs)
    assert np.all(np.abs(Ci[ok] - Cd[ok]) <= 1e-13 * S[ok])
    rows, cols = np.array([0, 36, 5]), np.array([28, 0, 7, 7])
    Cr, Sr = orc.gemm_dense(ac, as_, bc, bs, rows=rows)
    Cc, Sc = orc.gemm_dense(ac, as_, bc, bs, cols=cols)
    for got, want, sw in ((Cr, Cd[rows], Sd[rows]), (Cc, Cd[:, cols], Sd[:, cols])):
        assert np.array_equal(np.isnan(got), np.isnan(want))
        f = ~np.isnan(want)
        assert np.all(np.abs(got[f] - want[f]) <= 1e-13 * sw[f])


def test_hcp_residual_dense_equals_entries(orc):
    M, N, K = 24, 20, 256
    x = inputs.to_bf16_bits(inputs.normal((M, K), 31))
    w = inputs.to_bf16_bits(inputs.normal((K, N), 32, 0.02))
    hot = inputs.hot_channels(K, 33, 0.09)
    xq = orc.quantize(x, 32)
    wq = orc.quantize(w, 32, axis=orc.COL)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    R, S = orc.hcp_residual_entries(x, xq[0], xq[1], w, wq[0], wq[1], hot, ii.ravel(),
                                    jj.ravel())
    Rd, Sd = orc.hcp_residual_dense(x, xq[0], xq[1], w, wq[0], wq[1], hot)
    assert np.all(np.abs(R.reshape(M, N) - Rd) <= 1e-13 * Sd)
    assert np.allclose(S.reshape(M, N), Sd, rtol=1e-13, atol=0)
    rows, cols = np.array([23, 0, 4]), np.array([19, 3])
    Rr, Sr = orc.hcp_residual_dense(x, xq[0], xq[1], w, wq[0], wq[1], hot, rows=rows)
    Rc, Sc = orc.hcp_residual_dense(x, xq[0], xq[1], w, wq[0], wq[1], hot, cols=cols)
    assert np.allclose(Rr, Rd[rows], rtol=0, atol=1e-13 * Sd.max())
    assert np.allclose(Rc, Rd[:, cols], rtol=0, atol=1e-13 * Sd.max())


def test_hcp_split_dense_equals_entries(orc):
    M, N, K = 16, 12, 128
    x = inputs.to_bf16_bits(inputs.normal((M, K), 41))
    w = inputs.to_bf16_bits(inputs.normal((K, N), 42, 0.02))
    hot = inputs.hot_channels(K, 43, 0.1)
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    R, S = orc.hcp_split_entries(x, w, hot, ii.ravel(), jj.ravel())
    Rd, Sd = orc.hcp_split_dense(x, w, hot)
    assert np.allclose(R.reshape(M, N), Rd, rtol=0, atol=1e-13 * Sd.max())
    assert np.allclose(S.reshape(M, N), Sd, rtol=1e-13, atol=0)
    Rr, _ = orc.hcp_split_dense(x, w, hot, rows=np.array([15, 2]))
    Rc, _ = orc.hcp_split_dense(x, w, hot, cols=np.array([0, 11]))
    assert np.allclose(Rr, Rd[[15, 2]], rtol=0, atol=1e-13 * Sd.max())
    assert np.allclose(Rc, Rd[:, [0, 11]], rtol=0, atol=1e-13 * Sd.max())
