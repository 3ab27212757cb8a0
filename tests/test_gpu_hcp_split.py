"""GPU parity of the hot-channel compensation's split reading: the channel
mask (bit exact against the index list), the masked quantiser (bit exact
against the oracle's quantisation of the input with those channels zeroed,
and against fp4q_quantize of a zeroed copy), and fp4q_gemm_hcp_split (the
oracle's GEMM of the masked quantisations plus its split residual, within
the GEMM bound over the extended sum)."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import (check_gemm_f32, check_lines_f32, dev, dev_bf16, edge_lines,
                         host_bits, sample_positions)

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("length,n", [(1, 1), (37, 5), (5120, 461), (64, 64), (100, 0)])
def test_channel_mask(length, n):
    rng = np.random.default_rng(length + n)
    idx = np.sort(rng.choice(length, n, replace=False)).astype(np.int32)
    extra = np.array([-3, length, length + 40], np.int32)   # ignored, out of range
    m = fq.channel_mask(dev(np.concatenate([idx, extra])), length)
    torch.cuda.synchronize()
    want = np.zeros((length + 31) // 32, np.uint32)
    for c in idx:
        want[c >> 5] |= np.uint32(1 << (c & 31))
    assert np.array_equal(host_bits(m).view(np.uint32), want)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("axis", ["row", "col"])
@pytest.mark.parametrize("rounding", ["rne", "sr"])
def test_quantize_masked(orc, dtype, axis, rounding):
    R, C, block = 320, 416, 32
    x = inputs.with_outliers(inputs.normal((R, C), 71), 72, 300, 30.0)
    ax = fq.ROW if axis == "row" else fq.COL
    rnd = fq.RNE if rounding == "rne" else fq.SR
    length = C if axis == "row" else R
    hot = inputs.hot_channels(length, 73, 0.09)
    xz = x.copy()
    if axis == "row":
        xz[:, hot] = 0
    else:
        xz[hot, :] = 0
    if dtype == "bf16":
        xb, xzb = inputs.to_bf16_bits(x), inputs.to_bf16_bits(xz)
        xd, xzd = dev_bf16(xb), dev_bf16(xzb)
        ref = orc.quantize(xzb, block, axis=orc.ROW if ax == fq.ROW else orc.COL,
                           round=orc.RNE if rnd == fq.RNE else orc.SR, seed=9)
    else:
        xd, xzd = dev(x), dev(xz)
        ref = orc.quantize(xz, block, axis=orc.ROW if ax == fq.ROW else orc.COL,
                           round=orc.RNE if rnd == fq.RNE else orc.SR, seed=9)
    mask = fq.channel_mask(dev(hot), length)
    got = fq.quantize_masked(xd, mask, block, ax, rnd, 9)
    plain = fq.quantize(xzd, block, ax, rnd, 9)
    torch.cuda.synchronize()
    for g, p, r in zip(got, plain, ref):
        assert np.array_equal(g.cpu().numpy(), r)
        assert torch.equal(g, p)


# N a multiple of 8: the GPU quantiser takes 16-byte-aligned rows of W
@pytest.mark.parametrize("M,N,K,n_hot", [(64, 96, 256, 23), (300, 264, 512, 46), (64, 96, 192, 17),
                                         (1, 40, 128, 1), (128, 128, 256, 256),
                                         (96, 64, 128, 0)])
def test_gemm_hcp_split(orc, M, N, K, n_hot):
    x = inputs.to_bf16_bits(inputs.normal((M, K), M + K + 3))
    w = inputs.to_bf16_bits(inputs.normal((K, N), N + K + 3, 0.02))
    hot = inputs.hot_channels(K, 17, n_hot / K) if n_hot else np.zeros(0, np.int32)
    xz, wz = x.copy(), w.copy()
    xz[:, hot] = 0
    wz[hot, :] = 0
    xq = orc.quantize(xz, 32)
    wq = orc.quantize(wz, 32, axis=orc.COL)
    mask = fq.channel_mask(dev(hot), K)
    xqd = fq.quantize_masked(dev_bf16(x), mask, 32, fq.ROW)
    wqd = fq.quantize_masked(dev_bf16(w), mask, 32, fq.COL)
    y = fq.gemm_hcp_split(dev_bf16(x), xqd[0], xqd[1], dev_bf16(w), wqd[0], wqd[1], dev(hot))
    torch.cuda.synchronize()
    assert np.array_equal(xqd[0].cpu().numpy(), xq[0]) and np.array_equal(wqd[1].cpu().numpy(),
                                                                            wq[1])
    C, S = orc.gemm(xq[0], xq[1], wq[0], wq[1])
    ii, jj = np.meshgrid(np.arange(M), np.arange(N), indexing="ij")
    R, SR = orc.hcp_split_entries(x, w, hot, ii.ravel(), jj.ravel())
    check_gemm_f32(host_bits(y), C + R.reshape(M, N), S + SR.reshape(M, N),
                   f"hcp split {M}x{N}x{K} hot={n_hot}")


def test_outlier_layer_split(orc):
    """16384 x 13824 x 5120 with 461 hot channels, split reading: the masked
    quantisations of X and W bit for bit against the oracle's quantisations
    of the zeroed tensors (whole tensors), then the product on >= 4 sampled
    outputs per 128 x 128 tile and 64 whole rows and columns (first and last
    included)."""
    d = inputs.outlier_layer()
    X, W, hot = d["X"], d["W"], d["hot"]
    M, K = X.shape
    N = W.shape[1]
    xz = X.copy()
    xz[:, hot] = 0
    wz = W.copy()
    wz[hot, :] = 0
    A = orc.quantize(xz, 32)
    B = orc.quantize(wz, 32, axis=orc.COL)
    del xz, wz
    xd, wd, hd = dev_bf16(X), dev_bf16(W), dev(hot)
    mask = fq.channel_mask(hd, K)
    xq = fq.quantize_masked(xd, mask, 32, fq.ROW)
    wq = fq.quantize_masked(wd, mask, 32, fq.COL)
    y = fq.gemm_hcp_split(xd, xq[0], xq[1], wd, wq[0], wq[1], hd)
    torch.cuda.synchronize()
    for g, o, what in zip(xq + wq, A + B, ("X codes", "X scales", "W codes", "W scales")):
        assert np.array_equal(host_bits(g), o), what
    yh = host_bits(y)
    ii, jj = sample_positions(M, N, 8)
    C, S = orc.gemm_entries(A[0], A[1], B[0], B[1], ii, jj)
    R, SR = orc.hcp_split_entries(X, W, hot, ii, jj)
    check_gemm_f32(yh[ii, jj], C + R, S + SR, "13B split hcp")

    def ref(rows=None, cols=None):
        C, S = orc.gemm_dense(*A, *B, rows=rows, cols=cols)
        R, SR = orc.hcp_split_dense(X, W, hot, rows=rows, cols=cols)
        return C + R, S + SR
    check_lines_f32(orc, yh, edge_lines(M, 64, 81), edge_lines(N, 64, 82), ref, "13B split hcp")
