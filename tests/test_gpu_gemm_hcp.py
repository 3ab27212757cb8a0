"""GPU parity of fp4q_gemm (|c - C_ref| <= 1e-5 * sum|a_i b_i|; bf16 outputs
inside the rounded bracket) and fp4q_hcp_residual_add (same bound over the
extended sum): small/ragged sizes in full; the LLaMA-1B FFN GEMMs (forward
8192 x 5632 x 2048, dX 8192 x 2048 x 5632, dW 2048 x 5632 x 8192 with the DGE
estimator) over every output; the 13B-shaped outlier layer on >= 4 sampled
outputs per 128 x 128 tile plus 64 whole rows and 64 whole columns (the
first and last included)."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import (GEMM_REL, check_gemm_bf16, check_gemm_f32, check_lines_f32, dev,
                         dev_bf16, edge_lines, host_bits, sample_positions, to_dev_input)

pytestmark = pytest.mark.gpu


def qpair(orc, a, b):
    """Oracle ROW/block-32 quantisation of both operands (K-major)."""
    return orc.quantize(a, 32), orc.quantize(b, 32)


def gemm_full_check(orc, A, B, out_dtype=torch.float32, ldc_pad=0, accumulate=False, seed=0):
    (ac, as_), (bc, bs) = A, B
    M, N = ac.shape[0], bc.shape[0]
    C, S = orc.gemm(ac, as_, bc, bs)
    c = torch.full((M, N + ldc_pad), float("nan"), dtype=out_dtype, device="cuda")
    cv = c[:, :N]
    c0 = None
    if accumulate:
        c0 = inputs.normal((M, N), seed + 1)
        cv.copy_(torch.from_numpy(c0).cuda())
    fq.gemm(dev(ac), dev(as_), dev(bc), dev(bs), c=cv, accumulate=accumulate)
    torch.cuda.synchronize()
    full = host_bits(c)
    got = full[:, :N]
    if ldc_pad:
        pad = full[:, N:]
        assert (np.isnan(pad) if pad.dtype != np.uint16 else (pad & 0x7FFF) > 0x7F80).all(), \
            "gemm wrote past N"
    what = f"gemm M={M} N={N} K={2 * ac.shape[1]} {out_dtype} acc={accumulate}"
    if accumulate:
        C = C + c0
        S = S + np.abs(c0)
    if out_dtype == torch.bfloat16:
        check_gemm_bf16(got, C, S, orc, what)
    else:
        check_gemm_f32(got, C, S, what)


def test_tiny_ref_gemm(orc):
    d = inputs.tiny_ref()
    A, B = qpair(orc, d["A"], d["B"])
    gemm_full_check(orc, A, B)
    gemm_full_check(orc, A, B, torch.bfloat16)


TILES = ["256x256", "128x384"]


@pytest.mark.parametrize("tile", TILES)
@pytest.mark.parametrize("M,N,K", [(1, 1, 128), (300, 200, 256), (257, 129, 384),
                                   (64, 520, 128), (513, 33, 1024), (129, 769, 256),
                                   # K % 128 == 64: the K loop ends on a half step and the
                                   # scale rows are only 2-byte aligned
                                   (1, 1, 64), (300, 200, 192), (257, 129, 320),
                                   (129, 769, 64), (520, 300, 2112)])
def test_ragged_gemm(orc, M, N, K, tile, monkeypatch):
    monkeypatch.setenv("FP4Q_GEMM_TILE", tile)
    a = inputs.with_outliers(inputs.normal((M, K), M), M + 1, max(1, M * K // 100), 50.0)
    b = inputs.with_outliers(inputs.normal((N, K), N + 7), N + 8, max(1, N * K // 100), 50.0)
    A, B = qpair(orc, a, b)
    gemm_full_check(orc, A, B, torch.float32, ldc_pad=4)
    gemm_full_check(orc, A, B, torch.bfloat16, ldc_pad=8)
    gemm_full_check(orc, A, B, torch.float32, accumulate=True, seed=M)


@pytest.mark.parametrize("M,N,K", [(8192, 5632, 2048), (2048, 5632, 8192), (700, 1000, 512),
                                   (700, 1000, 576)])
def test_gemm_tiles_bit_identical(M, N, K, monkeypatch):
    """Both tile shapes accumulate each output over K in the same order: the
    outputs agree bit for bit (bf16 and fp32 C), including ragged edges."""
    rng = np.random.default_rng(M + N + K)
    ac = torch.from_numpy(rng.integers(0, 256, (M, K // 2), dtype=np.uint8)).cuda()
    bc = torch.from_numpy(rng.integers(0, 256, (N, K // 2), dtype=np.uint8)).cuda()
    as_ = torch.from_numpy(rng.integers(118, 136, (M, K // 32), dtype=np.uint8)).cuda()
    bs = torch.from_numpy(rng.integers(118, 136, (N, K // 32), dtype=np.uint8)).cuda()
    for dt in (torch.bfloat16, torch.float32):
        outs = []
        for tile in TILES:
            monkeypatch.setenv("FP4Q_GEMM_TILE", tile)
            outs.append(fq.gemm(ac, as_, bc, bs, out_dtype=dt))
        torch.cuda.synchronize()
        a = host_bits(outs[0])
        for t, o in zip(TILES[1:], outs[1:]):
            assert np.array_equal(a.view(np.uint8), host_bits(o).view(np.uint8)), \
                f"{M}x{N}x{K} {dt} {t}"


@pytest.mark.parametrize("M,N,K", [(64, 32, 128), (300, 288, 256), (513, 1056, 384),
                                   (300, 288, 320), (8192, 5632, 2048)])
def test_gemm_quant_epilogue(orc, M, N, K):
    """fp4q_gemm_quant against the oracle: its bf16 C inside the rounded
    bracket of the oracle's product (every output), and its codes and scales
    equal to the oracle's ROW block-32 nearest-even quantisation of that C;
    with and without the C store; bit for bit equal to fp4q_gemm then
    fp4q_quantize; a row of A whose scale byte is 0xFF gives a NaN row of C
    (scale 0xFF, codes 0).  Operands are the oracle's quantisations."""
    print(f"gemm_quant {M}x{N}x{K}", flush=True)
    a = inputs.normal((M, K), M + 11)
    b = inputs.normal((N, K), N + 13)
    (ac, as_), (bc, bs) = qpair(orc, a, b)
    as_ = as_.copy()
    as_[M // 2, 1] = 0xFF
    acd, asd, bcd, bsd = dev(ac), dev(as_), dev(bc), dev(bs)
    c, (qc, qs) = fq.gemm_quant(acd, asd, bcd, bsd)
    _, (qc2, qs2) = fq.gemm_quant(acd, asd, bcd, bsd, write_c=False)
    c_ref = fq.gemm(acd, asd, bcd, bsd, out_dtype=torch.bfloat16)
    qc_ref, qs_ref = fq.quantize(c_ref, 32, fq.ROW)
    torch.cuda.synchronize()
    cb = host_bits(c)
    C, S = orc.gemm_dense(ac, as_, bc, bs)
    nan = np.isnan(C)
    assert nan[M // 2].all() and nan.sum() == N
    assert ((cb[M // 2] & 0x7FFF) > 0x7F80).all()
    ok = ~nan.any(axis=1)
    check_gemm_bf16(cb[ok], C[ok], S[ok], orc, f"gemm_quant C {M}x{N}x{K}")
    oc, os_ = orc.quantize(cb, 32)
    for got_c, got_s in ((qc, qs), (qc2, qs2)):
        assert np.array_equal(host_bits(got_c), oc) and np.array_equal(host_bits(got_s), os_)
    assert (os_[M // 2] == 0xFF).all() and (oc[M // 2] == 0).all()
    assert torch.equal(c.view(torch.int16), c_ref.view(torch.int16))
    assert torch.equal(qc, qc_ref) and torch.equal(qs, qs_ref)


def test_gemm_nan_scale_and_zero(orc):
    a = inputs.normal((64, 256), 1)
    b = inputs.normal((64, 256), 2)
    (ac, as_), (bc, bs) = qpair(orc, a, b)
    as_ = as_.copy()
    as_[5, 3] = 0xFF
    ac[7] = 0
    c = fq.gemm(dev(ac), dev(as_), dev(bc), dev(bs), out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = host_bits(c)
    C, S = orc.gemm(ac, as_, bc, bs)
    assert np.isnan(got[5]).all()
    assert (got[7] == 0).all()
    ok = ~np.isnan(C)
    assert np.all(np.abs(got[ok] - C[ok]) <= GEMM_REL * S[ok])


def sampled_gemm_check(orc, A, B, c_gpu, seed, what):
    (ac, as_), (bc, bs) = A, B
    M, N = ac.shape[0], bc.shape[0]
    ii, jj = sample_positions(M, N, seed)
    C, S = orc.gemm_entries(ac, as_, bc, bs, ii, jj)
    got = host_bits(c_gpu)[ii, jj]
    if c_gpu.dtype == torch.bfloat16:
        check_gemm_bf16(got, C, S, orc, what)
    else:
        check_gemm_f32(got, C, S, what)
    return ii, jj, C, S


def test_ffn_forward_gemm(orc):
    """8192 x 5632 x 2048, bf16 and fp32 out, every output against the
    oracle; operands quantised on the GPU and checked bit-exact against the
    oracle's first."""
    d = inputs.ffn_forward()
    X, W = d["X"], d["W"]
    A = orc.quantize(X, 32)
    B = orc.quantize(W, 32, axis=orc.COL)
    xq = fq.quantize(dev_bf16(X), 32, fq.ROW)
    wq = fq.quantize(dev_bf16(W), 32, fq.COL)
    y = fq.gemm(xq[0], xq[1], wq[0], wq[1], out_dtype=torch.bfloat16)
    y32 = fq.gemm(xq[0], xq[1], wq[0], wq[1], out_dtype=torch.float32)
    torch.cuda.synchronize()
    for g, o in zip(xq + wq, A + B):
        assert np.array_equal(host_bits(g), o)
    C, S = orc.gemm_dense(*A, *B)
    check_gemm_bf16(host_bits(y), C, S, orc, "ffn fwd bf16")
    check_gemm_f32(host_bits(y32), C, S, "ffn fwd f32")


def test_ffn_backward_gemms_and_dge(orc):
    """dX = dY W^T (K = 5632, bf16) and dW = X^T dY (K = 8192, fp32) with dY
    stochastically rounded, then the DGE mask of W applied to dW (separately
    and in the GEMM's epilogue): every output against the oracle."""
    f = inputs.ffn_forward()
    b = inputs.ffn_backward_grad()
    X, W, dY = f["X"], f["W"], b["dY"]
    dyr = orc.quantize(dY, 32, round=orc.SR, seed=b["seed_row"])
    wr = orc.quantize(W, 32)
    dx = fq.gemm(dev(dyr[0]), dev(dyr[1]), dev(wr[0]), dev(wr[1]), out_dtype=torch.bfloat16)
    torch.cuda.synchronize()
    C, S = orc.gemm_dense(*dyr, *wr)
    check_gemm_bf16(host_bits(dx), C, S, orc, "dX")
    del dx, C, S
    xc = orc.quantize(X, 32, axis=orc.COL)
    dyc = orc.quantize(dY, 32, axis=orc.COL, round=orc.SR, seed=b["seed_col"])
    dw = fq.gemm(dev(xc[0]), dev(xc[1]), dev(dyc[0]), dev(dyc[1]), out_dtype=torch.float32)
    torch.cuda.synchronize()
    C, S = orc.gemm_dense(*xc, *dyc)
    check_gemm_f32(host_bits(dw), C, S, "dW")
    # DGE mask of W (COL blocks of 32) on the GPU's dW: out = dW * d, checked
    # against d_ref * C_ref with the GEMM bound and the DGE bound combined
    out = fq.grad_estimate(fq.DGE, dev_bf16(W), dw, 32, fq.COL, 5.0, 3.0,
                           out_dtype=torch.float32)
    torch.cuda.synchronize()
    d_ref, _ = orc.grad_estimate(orc.DGE, W, np.zeros(W.shape, np.float32), 32, orc.COL)
    got = host_bits(out).astype(np.float64)
    tol = d_ref * (GEMM_REL * S) * (1 + 2.0 ** -20) + np.abs(C) * d_ref * 2.0 ** -20 \
        + np.abs(C * d_ref) * 2.0 ** -23
    assert np.all(np.abs(got - C * d_ref) <= tol)
    # the same product from the GEMM with the estimator in its epilogue
    fused = fq.gemm_dge(dev(xc[0]), dev(xc[1]), dev(dyc[0]), dev(dyc[1]), dev_bf16(W), 5.0, 3.0)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(fused).view(np.uint32), host_bits(out).view(np.uint32)), \
        "gemm_dge differs from gemm + grad_estimate"


@pytest.mark.parametrize("M,N,K,k", [(32, 1, 128, 5.0), (96, 200, 256, 5.0), (320, 517, 384, 5.0),
                                     (96, 200, 192, 5.0), (64, 70, 64, 3.0),
                                     (256, 256, 512, 1.0), (64, 388, 128, 3.0)])
def test_gemm_dge_small(orc, M, N, K, k):
    """fp4q_gemm_dge against the oracle (GEMM entries times the oracle's DGE
    derivative of x, COL blocks of 32) over every output, and bit for bit
    against fp4q_gemm + fp4q_grad_estimate; x carries a zero block, a block
    with an Inf (its outputs are NaN) and outliers."""
    a = inputs.normal((M, K), M + 3)
    b = inputs.normal((N, K), N + 5)
    A, B = qpair(orc, a, b)
    x = inputs.with_outliers(inputs.normal((M, N), M + N, 0.02), 9, max(1, M * N // 100), 50.0)
    x[0:32, 0] = 0.0
    if N > 2:
        x[5, 2] = np.inf
    xb = inputs.to_bf16_bits(x)
    out = fq.gemm_dge(dev(A[0]), dev(A[1]), dev(B[0]), dev(B[1]), dev_bf16(xb), k, 3.0)
    g = fq.gemm(dev(A[0]), dev(A[1]), dev(B[0]), dev(B[1]), out_dtype=torch.float32)
    two = fq.grad_estimate(fq.DGE, dev_bf16(xb), g, 32, fq.COL, k, 3.0, out_dtype=torch.float32)
    torch.cuda.synchronize()
    got = host_bits(out).astype(np.float64)
    assert np.array_equal(host_bits(out).view(np.uint32), host_bits(two).view(np.uint32))
    C, S = orc.gemm(A[0], A[1], B[0], B[1])
    d_ref, _ = orc.grad_estimate(orc.DGE, xb, np.zeros((M, N), np.float32), 32, orc.COL, k, 3.0)
    nan = np.isnan(d_ref)
    assert np.isnan(got[nan]).all()
    if N > 2:
        assert nan[0:32, 2].all() and not nan[32:, 2].any()
    ok = ~nan
    tol = d_ref[ok] * (GEMM_REL * S[ok]) * (1 + 2.0 ** -20) + np.abs(C[ok]) * d_ref[ok] * 2.0 ** -20 \
        + np.abs(C[ok] * d_ref[ok]) * 2.0 ** -23
    assert np.all(np.abs(got[ok] - C[ok] * d_ref[ok]) <= tol)


def _outlier_refs(orc, X, A, W, B, hot):
    """Oracle references of the 13B-shaped layer for whole lines: the base
    product, and the base product plus the hot-channel residual."""
    def base(rows=None, cols=None):
        return orc.gemm_dense(*A, *B, rows=rows, cols=cols)

    def with_hcp(rows=None, cols=None):
        C, S = orc.gemm_dense(*A, *B, rows=rows, cols=cols)
        R, SR = orc.hcp_residual_dense(X, A[0], A[1], W, B[0], B[1], hot, rows=rows, cols=cols)
        return C + R, S + SR
    return base, with_hcp


def test_outlier_layer_gemm_and_hcp(orc):
    """16384 x 13824 x 5120 fp32 base GEMM plus the dual-mode hot-channel
    residual over 9% persistent hot channels: >= 4 sampled outputs per
    128 x 128 tile and 64 whole rows and columns (first and last included),
    before and after the residual add."""
    d = inputs.outlier_layer()
    X, W, hot = d["X"], d["W"], d["hot"]
    A = orc.quantize(X, 32)
    B = orc.quantize(W, 32, axis=orc.COL)
    Ad = (dev(A[0]), dev(A[1]))
    Bd = (dev(B[0]), dev(B[1]))
    y = fq.gemm(Ad[0], Ad[1], Bd[0], Bd[1], out_dtype=torch.float32)
    torch.cuda.synchronize()
    M, N = y.shape
    yh = host_bits(y)
    ii, jj = sample_positions(M, N, 7)
    C, S = orc.gemm_entries(A[0], A[1], B[0], B[1], ii, jj)
    check_gemm_f32(yh[ii, jj], C, S, "13B base")
    rows, cols = edge_lines(M, 64, 71), edge_lines(N, 64, 72)
    base, with_hcp = _outlier_refs(orc, X, A, W, B, hot)
    check_lines_f32(orc, yh, rows, cols, base, "13B base")
    xd, wd = dev_bf16(X), dev_bf16(W)
    fq.hcp_residual_add(xd, Ad[0], Ad[1], wd, Bd[0], Bd[1], dev(hot), y)
    torch.cuda.synchronize()
    yh = host_bits(y)
    R, SR = orc.hcp_residual_entries(X, A[0], A[1], W, B[0], B[1], hot, ii, jj)
    check_gemm_f32(yh[ii, jj], C + R, S + SR, "13B base + hcp")
    check_lines_f32(orc, yh, rows, cols, with_hcp, "13B base + hcp")


@pytest.mark.parametrize("M,N,K,n_hot", [(64, 96, 256, 23), (300, 257, 512, 46),
                                         (1, 33, 128, 1), (128, 128, 256, 256),
                                         # X's rows too long to stage in LDS (its gather
                                         # reads global memory directly), W's staged
                                         (64, 40, 16384, 37),
                                         # both staged, several hundred hot channels
                                         (48, 40, 8192, 500),
                                         # three X rows per workgroup, the last one ragged
                                         (50, 40, 1024, 70),
                                         # rows too long to stage for either gather
                                         (16, 24, 20480, 61)])
def test_hcp_small(orc, M, N, K, n_hot):
    x = inputs.to_bf16_bits(inputs.normal((M, K), M + K))
    w = inputs.to_bf16_bits(inputs.normal((K, N), N + K, 0.02))
    hot = inputs.hot_channels(K, 11, n_hot / K)
    assert hot.size == n_hot
    x64 = x.copy()
    xq = orc.quantize(x, 32)
    wq = orc.quantize(w, 32, axis=orc.COL)
    y0 = inputs.normal((M, N), 12)
    y = dev(y0.copy())
    fq.hcp_residual_add(dev_bf16(x), dev(xq[0]), dev(xq[1]), dev_bf16(w), dev(wq[0]),
                        dev(wq[1]), dev(hot), y)
    torch.cuda.synchronize()
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    ii, jj = ii.ravel(), jj.ravel()
    R, S = orc.hcp_residual_entries(x64, xq[0], xq[1], w, wq[0], wq[1], hot, ii, jj)
    want = y0.astype(np.float64).ravel() + R
    check_gemm_f32(host_bits(y).ravel(), want, S + np.abs(y0).ravel(), f"hcp {M}x{N}x{K}")


def test_hcp_empty_is_noop(orc):
    x = inputs.to_bf16_bits(inputs.normal((32, 64), 1))
    w = inputs.to_bf16_bits(inputs.normal((64, 32), 2))
    xq = orc.quantize(x, 32)
    wq = orc.quantize(w, 32, axis=orc.COL)
    y0 = inputs.normal((32, 32), 3)
    y = dev(y0.copy())
    fq.hcp_residual_add(dev_bf16(x), dev(xq[0]), dev(xq[1]), dev_bf16(w), dev(wq[0]),
                        dev(wq[1]), torch.zeros(0, dtype=torch.int32, device="cuda"), y)
    torch.cuda.synchronize()
    assert np.array_equal(host_bits(y), y0)


@pytest.mark.parametrize("M,N,K,n_hot,ld_pad", [(64, 96, 256, 23, 0), (300, 257, 512, 46, 3),
                                                (64, 96, 320, 29, 1), (33, 65, 64, 6, 0),
                                                (1, 33, 128, 1, 0), (128, 128, 256, 256, 0),
                                                (513, 260, 384, 0, 1), (64, 40, 16384, 37, 0),
                                                (48, 40, 8192, 500, 2)])
def test_gemm_hcp_single_kernel(orc, M, N, K, n_hot, ld_pad):
    """fp4q_gemm_hcp: Y = Xq Wq + residual in one kernel, against the oracle's
    base GEMM plus its residual entries, over the sum of both bounds; columns
    past N (ld_y padding) stay untouched."""
    x = inputs.to_bf16_bits(inputs.normal((M, K), M + K + 1))
    w = inputs.to_bf16_bits(inputs.normal((K, N), N + K + 1, 0.02))
    hot = inputs.hot_channels(K, 13, n_hot / K) if n_hot else np.zeros(0, np.int32)
    assert hot.size == n_hot
    xq = orc.quantize(x, 32)
    wq = orc.quantize(w, 32, axis=orc.COL)
    C, S = orc.gemm(xq[0], xq[1], wq[0], wq[1])
    y = torch.full((M, N + ld_pad), float("nan"), dtype=torch.float32, device="cuda")
    fq.gemm_hcp(dev_bf16(x), dev(xq[0]), dev(xq[1]), dev_bf16(w), dev(wq[0]), dev(wq[1]),
                dev(hot), y=y[:, :N])
    torch.cuda.synchronize()
    full = host_bits(y)
    if ld_pad:
        assert np.isnan(full[:, N:]).all(), "gemm_hcp wrote past N"
    got = full[:, :N]
    if n_hot:
        ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
        R, SR = orc.hcp_residual_entries(x, xq[0], xq[1], w, wq[0], wq[1], hot, ii.ravel(),
                                         jj.ravel())
        C = C + R.reshape(M, N)
        S = S + SR.reshape(M, N)
    check_gemm_f32(got, C, S, f"gemm_hcp {M}x{N}x{K} hot={n_hot}")


def test_outlier_layer_single_kernel_hcp(orc):
    """16384 x 13824 x 5120 with 461 hot channels in one kernel: >= 4 sampled
    outputs per 128 x 128 tile and 64 whole rows and columns (first and last
    included), and equal to the two-call form within the same bound."""
    d = inputs.outlier_layer()
    X, W, hot = d["X"], d["W"], d["hot"]
    A = orc.quantize(X, 32)
    B = orc.quantize(W, 32, axis=orc.COL)
    Ad = (dev(A[0]), dev(A[1]))
    Bd = (dev(B[0]), dev(B[1]))
    xd, wd, hd = dev_bf16(X), dev_bf16(W), dev(hot)
    y = fq.gemm_hcp(xd, Ad[0], Ad[1], wd, Bd[0], Bd[1], hd)
    torch.cuda.synchronize()
    M, N = y.shape
    yh = host_bits(y)
    ii, jj = sample_positions(M, N, 7)
    C, S = orc.gemm_entries(A[0], A[1], B[0], B[1], ii, jj)
    R, SR = orc.hcp_residual_entries(X, A[0], A[1], W, B[0], B[1], hot, ii, jj)
    check_gemm_f32(yh[ii, jj], C + R, S + SR, "13B single-kernel hcp")
    _, with_hcp = _outlier_refs(orc, X, A, W, B, hot)
    check_lines_f32(orc, yh, edge_lines(M, 64, 73), edge_lines(N, 64, 74), with_hcp,
                    "13B single-kernel hcp")
    y2 = fq.gemm(Ad[0], Ad[1], Bd[0], Bd[1], out_dtype=torch.float32)
    fq.hcp_residual_add(xd, Ad[0], Ad[1], wd, Bd[0], Bd[1], hd, y2)
    torch.cuda.synchronize()
    a, b = yh[ii, jj].astype(np.float64), host_bits(y2)[ii, jj].astype(np.float64)
    assert np.all(np.abs(a - b) <= 2 * GEMM_REL * (S + SR)), "single-kernel vs two-call"


@pytest.mark.parametrize("M,N,K,grid", [(700, 1000, 2048, 5), (257, 513, 4096, 2),
                                        (1024, 1024, 2048, 7), (300, 260, 2048, 1),
                                        (300, 520, 3072, 3), (260, 300, 5120, 1)])
def test_persistent_gemm_chains_tiles(orc, M, N, K, grid, monkeypatch):
    """The persistent form (one workgroup walking several tiles, the operand
    ring running on across tile boundaries) against the oracle over every
    output, bf16, fp32 and accumulated fp32, with fewer workgroups than tiles
    so that each chains several; and bit for bit equal to the
    one-tile-per-workgroup kernel.  K = 3072 and 5120 end each tile on a half
    turn of the K loop, so the tiles' first scale buffers alternate (four
    tiles on one workgroup at 260 x 300 x 5120)."""
    a = inputs.with_outliers(inputs.normal((M, K), M + 31), M + 32, M * K // 100, 50.0)
    b = inputs.with_outliers(inputs.normal((N, K), N + 33), N + 34, N * K // 100, 50.0)
    A, B = qpair(orc, a, b)
    monkeypatch.setenv("FP4Q_GEMM_TILE", "256x256")
    monkeypatch.setenv("FP4Q_GEMM_PERSIST", "1")
    monkeypatch.setenv("FP4Q_GEMM_PERSIST_GRID", str(grid))
    gemm_full_check(orc, A, B, torch.float32, ldc_pad=4)
    gemm_full_check(orc, A, B, torch.bfloat16, ldc_pad=8)
    gemm_full_check(orc, A, B, torch.float32, accumulate=True, seed=M)
    ad, asd, bd, bsd = dev(A[0]), dev(A[1]), dev(B[0]), dev(B[1])
    for dt in (torch.bfloat16, torch.float32):
        monkeypatch.setenv("FP4Q_GEMM_PERSIST", "1")
        p = fq.gemm(ad, asd, bd, bsd, out_dtype=dt)
        monkeypatch.setenv("FP4Q_GEMM_PERSIST", "0")
        q = fq.gemm(ad, asd, bd, bsd, out_dtype=dt)
        torch.cuda.synchronize()
        assert np.array_equal(host_bits(p).view(np.uint8), host_bits(q).view(np.uint8)), dt

