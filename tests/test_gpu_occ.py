"""GPU parity of the outlier clamping and compensation (fp4q_occ_quantize,
fp4q_occ_spmm): the threshold, the clamped quantisation (codes and scales)
and the residual CSR (row pointers, columns, fp32 values) bit for bit against
the oracle, nearest-even and stochastic, over quantiles, ragged shapes, a
padded row stride, Inf/NaN elements and the LLaMA-1B FFN activation; the
sparse product within the GEMM bound (untouched rows bit for bit); and the
compensated layer output Xq Wq + R W against the oracle."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import (GEMM_REL, assert_float_bits_equal, assert_same_bits, dev, dev_bf16,
                         host_bits)

pytestmark = pytest.mark.gpu


def t_bits(t):
    return int(np.float32(t).view(np.uint32) >> 16)


def run_and_check(orc, xb, xd, q, rnd, seed=0, off=0):
    print(f"occ_quantize shape={xb.shape} ld={xd.stride(0)} q={q} round={rnd} seed={seed}",
          flush=True)
    r = fq.RNE if rnd == "rne" else fq.SR
    codes, scales, rp, ci, v, thr = fq.occ_quantize(xd, q, r, seed, off)
    torch.cuda.synchronize()
    t, nnz = orc.occ_threshold(xb, q)
    clamped, rp_w, ci_w, v_w = orc.occ_split(xb, t)
    assert int(host_bits(thr).view(np.uint16)[0]) == t_bits(t)
    wc, ws = orc.quantize(clamped, 32, orc.ROW, orc.RNE if rnd == "rne" else orc.SR, seed, off)
    assert_same_bits(host_bits(codes), wc, "codes")
    assert_same_bits(host_bits(scales), ws, "scales")
    hp = host_bits(rp)
    assert_same_bits(hp, rp_w, "row_ptr")
    assert hp[-1] == nnz <= fq.occ_max_nnz(*xb.shape, q)
    assert_same_bits(host_bits(ci)[:nnz], ci_w, "col_idx")
    assert_float_bits_equal(host_bits(v)[:nnz], v_w, "vals")
    return codes, scales, rp, ci, v


@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("shape,q", [((1, 32), 0.99), ((37, 96), 0.99), ((130, 416), 0.9),
                                     ((64, 2048), 0.99), ((300, 160), 0.5), ((50, 64), 1.0),
                                     # more rows than the row-count scan stages in LDS
                                     ((8200, 32), 0.99)])
def test_occ_quantize_parity(orc, shape, q, rnd):
    xb = inputs.to_bf16_bits(inputs.with_outliers(inputs.student_t(shape, shape[0] + 7), 11,
                                                  max(1, shape[0] * shape[1] // 150), 30.0))
    run_and_check(orc, xb, dev_bf16(xb), q, rnd, seed=77 + shape[0], off=shape[1])


def test_occ_quantize_stride_and_nonfinite(orc):
    wide = inputs.to_bf16_bits(inputs.normal((90, 192 + 32), 991))
    wide[4, 32 + 10] = 0x7F80          # +inf
    wide[60, 32 + 100] = 0xFF80        # -inf
    wide[33, 32 + 7] = 0xFFC1          # NaN
    xd = dev_bf16(wide)[:, 32:]
    xb = np.ascontiguousarray(wide[:, 32:])
    for rnd in ("rne", "sr"):
        run_and_check(orc, xb, xd, 0.99, rnd, seed=3)
    nan = np.full((8, 32), 0x7FC0, np.uint16)   # T is NaN: nothing clamped
    nan[0, :4] = 0x3F80
    run_and_check(orc, nan, dev_bf16(nan), 0.99, "rne")


def test_occ_quantize_ffn_activation(orc):
    # the LLaMA-1B FFN input shape with heavy-tailed activations (the
    # activation-sweep distribution): 16.8 M elements, 1% clamped
    xb = inputs.to_bf16_bits(inputs.student_t((8192, 2048), 992))
    run_and_check(orc, xb, dev_bf16(xb), 0.99, "rne")


@pytest.mark.parametrize("M,N,K,q", [(16, 64, 128, 0.9), (130, 200, 512, 0.99),
                                     (256, 1032, 384, 0.95)])
def test_occ_spmm_and_layer(orc, M, N, K, q):
    xb = inputs.to_bf16_bits(inputs.with_outliers(inputs.student_t((M, K), 993), 994, M, 40.0))
    wb = inputs.to_bf16_bits(inputs.normal((K, N), 995, 0.02))
    xd, wd = dev_bf16(xb), dev_bf16(wb)
    codes, scales, rp, ci, v, _ = fq.occ_quantize(xd, q)
    y0 = torch.from_numpy(inputs.normal((M, N), 996)).cuda()
    y = y0.clone()
    print(f"occ_spmm M={M} N={N} K={K}", flush=True)
    fq.occ_spmm(rp, ci, v, wd, y)
    torch.cuda.synchronize()
    hp, hc, hv = host_bits(rp), host_bits(ci), host_bits(v)
    res, mag = orc.occ_spmm(hp, hc[:hp[-1]], hv[:hp[-1]], wb)
    got = host_bits(y).astype(np.float64)
    base = host_bits(y0).astype(np.float64)
    err = np.abs(got - (base + res))
    bound = GEMM_REL * (mag + np.abs(base)) + 1e-30
    assert np.all(err <= bound), float((err / bound).max())
    empty = np.diff(hp) == 0
    assert np.array_equal(got[empty], base[empty])
    # the compensated layer: Xq Wq (clamped activation) + R W
    wq = fq.quantize(wd, 32, fq.COL)
    yl = fq.gemm(codes, scales, wq[0], wq[1], out_dtype=torch.float32)
    fq.occ_spmm(rp, ci, v, wd, yl)
    torch.cuda.synchronize()
    t, _ = orc.occ_threshold(xb, q)
    clamped, rp_w, ci_w, v_w = orc.occ_split(xb, t)
    xc, xs = orc.quantize(clamped, 32)
    wc, wsc = orc.quantize(wb, 32, orc.COL)
    C, S = orc.gemm(xc, xs, wc, wsc)
    r2, m2 = orc.occ_spmm(rp_w, ci_w, v_w, wb)
    err = np.abs(host_bits(yl).astype(np.float64) - (C + r2))
    assert np.all(err <= GEMM_REL * (S + m2) + 1e-30)


def test_occ_reconstruction_with_identity(orc):
    """The compensated reconstruction the benchmark's fidelity context uses:
    the dequantised clamped codes plus R I (fp4q_occ_spmm with a bf16
    identity) equals the oracle's dequantised clamp plus its residual, each
    entry to one fp32 rounding; and it is closer to x than the direct
    quantisation in cosine, MSE and SNR (heavy-tailed input)."""
    xb = inputs.to_bf16_bits(inputs.student_t((256, 512), 77))
    xd = dev_bf16(xb)
    codes, scales, rp, ci, v = run_and_check(orc, xb, xd, 0.99, "rne")
    comp = fq.dequantize(codes, scales, 32, torch.float32)
    fq.occ_spmm(rp, ci, v, torch.eye(512, dtype=torch.bfloat16, device="cuda"), comp)
    direct = fq.dequantize(*fq.quantize(xd, 32), 32, torch.float32)
    torch.cuda.synchronize()
    t, _ = orc.occ_threshold(xb, 0.99)
    clamped, rp_w, ci_w, v_w = orc.occ_split(xb, t)
    want = orc.dequantize(*orc.quantize(clamped, 32), 32)
    rows = np.repeat(np.arange(xb.shape[0]), np.diff(rp_w))
    want[rows, ci_w] += v_w.astype(np.float64)
    got = host_bits(comp).astype(np.float64)
    assert np.all(np.abs(got - want) <= np.abs(want) * 2.0 ** -24)
    x = (xb.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    dh = host_bits(direct).astype(np.float64)
    cos = lambda a: (a * x).sum() / np.linalg.norm(a) / np.linalg.norm(x)
    err = lambda a: ((a - x) ** 2).sum()
    assert cos(got) > cos(dh) and err(got) < err(dh)
