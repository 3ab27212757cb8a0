"""fp4q_hcp_residual_add_noalloc (the hot-channel residual add without a
caller workspace, for callers that cannot allocate): called through the C ABI
twice in a row -- first at the 13B-shaped outlier layer (16384 x 13824,
K = 5120, 461 hot channels: 56 MB of the 64 MiB library scratch), then at a
smaller ragged size -- each time bit for bit equal to fp4q_hcp_residual_add
with a caller workspace (the same kernels), and the small call also within
the oracle's bound."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import check_gemm_f32, dev, dev_bf16, host_bits

pytestmark = pytest.mark.gpu


def _both(x, xq, w, wq, hot, y0):
    """(noalloc result, workspace result) from the same starting y."""
    y1 = y0.clone()
    y2 = y0.clone()
    fq.hcp_residual_add_noalloc(x, xq[0], xq[1], w, wq[0], wq[1], hot, y1)
    fq.hcp_residual_add(x, xq[0], xq[1], w, wq[0], wq[1], hot, y2)
    torch.cuda.synchronize()
    return y1, y2


def test_noalloc_matches_workspace_call_large_then_small(orc):
    print("noalloc call 1: 16384 x 13824 x 5120, 461 hot", flush=True)
    d = inputs.outlier_layer()
    X, W, hot = d["X"], d["W"], d["hot"]
    M, K = X.shape
    N = W.shape[1]
    assert fq.hcp_workspace_bytes(M, N, hot.size) <= fq.HCP_NOALLOC_MAX_BYTES
    xd, wd, hd = dev_bf16(X), dev_bf16(W), dev(hot)
    xq = fq.quantize(xd, 32, fq.ROW)
    wq = fq.quantize(wd, 32, fq.COL)
    y0 = torch.from_numpy(inputs.normal((M, N), 5)).cuda()
    y1, y2 = _both(xd, xq, wd, wq, hd, y0)
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), "large call"
    del xd, wd, xq, wq, y0, y1, y2, X, W, d
    torch.cuda.empty_cache()

    print("noalloc call 2: 300 x 257 x 512, 46 hot", flush=True)
    M, N, K, n_hot = 300, 257, 512, 46
    x = inputs.to_bf16_bits(inputs.normal((M, K), 61))
    w = inputs.to_bf16_bits(inputs.normal((K, N), 62, 0.02))
    hot = inputs.hot_channels(K, 63, n_hot / K)
    xq = orc.quantize(x, 32)
    wq = orc.quantize(w, 32, axis=orc.COL)
    y0h = inputs.normal((M, N), 64)
    y1, y2 = _both(dev_bf16(x), (dev(xq[0]), dev(xq[1])), dev_bf16(w), (dev(wq[0]), dev(wq[1])),
                   dev(hot), torch.from_numpy(y0h).cuda())
    assert torch.equal(y1.view(torch.int32), y2.view(torch.int32)), "small call"
    R, S = orc.hcp_residual_dense(x, xq[0], xq[1], w, wq[0], wq[1], hot)
    check_gemm_f32(host_bits(y1), y0h.astype(np.float64) + R, S + np.abs(y0h), "noalloc small")


def test_noalloc_rejects_sizes_beyond_the_scratch():
    M, N, n_hot = 65536, 65536, 64     # (M + N) * 128 * 2 bytes = 32 MiB: fits
    assert fq.hcp_workspace_bytes(M, N, n_hot) <= fq.HCP_NOALLOC_MAX_BYTES
    M = 1 << 20                        # (2^20 + 2^16) * 128 * 2 bytes > 64 MiB
    assert fq.hcp_workspace_bytes(M, N, n_hot) > fq.HCP_NOALLOC_MAX_BYTES
    x = torch.zeros((64,), dtype=torch.bfloat16, device="cuda")
    u8 = torch.zeros((64,), dtype=torch.uint8, device="cuda")
    hot = torch.zeros((n_hot,), dtype=torch.int32, device="cuda")
    y = torch.zeros((16,), dtype=torch.float32, device="cuda")
    L = fq.lib()
    st = L.fp4q_hcp_residual_add_noalloc(M, N, 1024, fq._ptr(x), fq._ptr(u8), fq._ptr(u8),
                                         fq._ptr(x), fq._ptr(u8), fq._ptr(u8), fq._ptr(hot),
                                         n_hot, fq._ptr(y), None)
    assert st == 4 and b"static maximum" in L.fp4q_last_error()
