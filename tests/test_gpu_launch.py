"""fp4q_set_next_launch on the GPU: events recorded by a kernel's own
dispatch (the GEMM's, plain and persistent forms) and any-order launches of
independent kernels, whose outputs must equal a sequential run's bit for bit
(the linear layer's forward and backward step at a reduced size)."""
import ctypes
import os

import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import host_bits

pytestmark = pytest.mark.gpu


def hip_lib():
    return ctypes.CDLL(os.path.join(os.path.dirname(torch.__file__), "lib", "libamdhip64.so"))


@pytest.mark.parametrize("M,N,K", [(1024, 768, 2048), (4096, 5632, 2048)])
def test_gemm_dispatch_events(M, N, K):
    """fp4q_set_next_launch with events: the next GEMM launch (one tile per workgroup at
    1024 x 768, the persistent form at 4096 x 5632) records the pair at its
    own dispatch; its output is the plain launch's bit for bit, and the pair
    is used once (the launch after it is plain and leaves the events alone)."""
    hip = hip_lib()
    ev = [ctypes.c_void_p(), ctypes.c_void_p()]
    for e in ev:
        assert hip.hipEventCreateWithFlags(ctypes.byref(e), 0) == 0
    try:
        rng = np.random.default_rng(M + N)
        ac = torch.from_numpy(rng.integers(0, 256, (M, K // 2), dtype=np.uint8)).cuda()
        bc = torch.from_numpy(rng.integers(0, 256, (N, K // 2), dtype=np.uint8)).cuda()
        as_ = torch.from_numpy(rng.integers(118, 136, (M, K // 32), dtype=np.uint8)).cuda()
        bs = torch.from_numpy(rng.integers(118, 136, (N, K // 32), dtype=np.uint8)).cuda()
        plain = fq.gemm(ac, as_, bc, bs)
        fq.set_next_launch(ev[0], ev[1])
        timed = fq.gemm(ac, as_, bc, bs)
        torch.cuda.synchronize()
        ms = ctypes.c_float()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        first = ms.value
        assert 0.0 < first < 1000.0, first
        after = fq.gemm(ac, as_, bc, bs)
        torch.cuda.synchronize()
        assert hip.hipEventElapsedTime(ctypes.byref(ms), ev[0], ev[1]) == 0
        assert ms.value == first, "a plain launch re-recorded the events"
        for o in (timed, after):
            assert np.array_equal(host_bits(o).view(np.uint8), host_bits(plain).view(np.uint8))
        fq.set_next_launch()
    finally:
        for e in ev:
            hip.hipEventDestroy(e)


@pytest.mark.parametrize("M,K,N", [(1024, 512, 768), (2048, 1024, 1408)])
def test_any_order_step_matches_sequential(M, K, N):
    """The FFN step with the quantisers of W and dY, dequantize and the two
    backward GEMMs launched any-order (as the benchmark does) writes the same
    bits as the step with every launch behind a barrier, over three steps in
    a row on the same buffers."""
    f = inputs.ffn_forward(M, K, N)
    g = inputs.ffn_backward_grad(M, N)

    def bf16(bits):
        return torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).cuda()

    X, W, dY = bf16(f["X"]), bf16(f["W"]), bf16(g["dY"])
    u8 = dict(dtype=torch.uint8, device="cuda")
    b = {"xr": (torch.empty((M, K // 2), **u8), torch.empty((M, K // 32), **u8)),
         "wc": (torch.empty((N, K // 2), **u8), torch.empty((N, K // 32), **u8)),
         "dyr": (torch.empty((M, N // 2), **u8), torch.empty((M, N // 32), **u8)),
         "wr": (torch.empty((K, N // 2), **u8), torch.empty((K, N // 32), **u8)),
         "xc": (torch.empty((K, M // 2), **u8), torch.empty((K, M // 32), **u8)),
         "dyc": (torch.empty((N, M // 2), **u8), torch.empty((N, M // 32), **u8))}
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Xdq = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dX = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    dW = torch.empty((K, N), dtype=torch.float32, device="cuda")

    def dual(t, r, seed, a, c):
        fq.quantize_dual(t, 32, r, seed, r, seed, out=(b[a][0], b[a][1], b[c][0], b[c][1]))

    step = [(False, lambda: dual(X, fq.RNE, 0, "xr", "xc")),
            (True, lambda: dual(W, fq.RNE, 0, "wr", "wc")),
            (True, lambda: dual(dY, fq.SR, 1234, "dyr", "dyc")),
            (False, lambda: fq.gemm(*b["xr"], *b["wc"], c=Y)),
            (True, lambda: fq.dequantize(*b["xr"], 32, out=Xdq)),
            (True, lambda: fq.gemm(*b["dyr"], *b["wr"], c=dX)),
            (True, lambda: fq.gemm_dge(*b["xc"], *b["dyc"], W, 5.0, 3.0, out=dW))]
    outs = lambda: [t.clone() for k in b for t in b[k]] + [Y.clone(), Xdq.clone(), dX.clone(),
                                                           dW.clone()]
    for _, fn in step:
        fn()
    torch.cuda.synchronize()
    ref = outs()
    for t in [t for k in b for t in b[k]] + [Y, Xdq, dX, dW]:
        t.zero_()
    for _ in range(3):
        for ao, fn in step:
            if ao:
                fq.set_next_launch(any_order=True)
            fn()
    torch.cuda.synchronize()
    for i, (r, o) in enumerate(zip(ref, outs())):
        assert torch.equal(r.view(torch.uint8), o.view(torch.uint8)), f"output {i}"
