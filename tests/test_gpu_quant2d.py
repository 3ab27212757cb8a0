"""GPU parity of the two-dimensional block scaling (fp4q_quantize_2d): codes
and scales in both layouts bit for bit against the oracle, nearest-even and
stochastic, over ragged region counts, a padded row stride, a non-finite
square and the LLaMA-1B FFN weight shape; the two layouts dequantise to one
matrix and its transpose."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import assert_same_bits, dev_bf16, host_bits

pytestmark = pytest.mark.gpu

NAMES = ("row_codes", "row_scales", "col_codes", "col_scales")


def check(orc, xb, xd, rnd, seed=0, off=0):
    print(f"quantize_2d shape={xb.shape} ld={xd.stride(0)} round={rnd} seed={seed} off={off}",
          flush=True)
    r = fq.RNE if rnd == "rne" else fq.SR
    got = fq.quantize_2d(xd, r, seed, off)
    torch.cuda.synchronize()
    want = orc.quantize_2d(xb, 32, orc.RNE if rnd == "rne" else orc.SR, seed, off)
    for n, g, w in zip(NAMES, got, want):
        assert_same_bits(host_bits(g), w, n)
    return got


@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("shape", [(32, 32), (96, 160), (128, 128), (288, 416), (160, 4128)])
def test_quantize_2d_parity(orc, rnd, shape):
    xb = inputs.to_bf16_bits(inputs.with_outliers(inputs.student_t(shape, sum(shape)), 5,
                                                  max(1, shape[0] * shape[1] // 300), 30.0))
    check(orc, xb, dev_bf16(xb), rnd, seed=1234 + shape[1], off=7 * shape[0])


def test_quantize_2d_row_stride_nonfinite_and_one_matrix(orc):
    wide = inputs.to_bf16_bits(inputs.normal((192, 256 + 96), 941))
    wide[70, 96 + 40] = 0x7F80        # +inf: square (2, 1) of the view
    wide[5, 96 + 200] = 0xFFC0        # NaN: square (0, 6)
    xd = dev_bf16(wide)[:, 96:]
    xb = np.ascontiguousarray(wide[:, 96:])
    for rnd in ("rne", "sr"):
        got = check(orc, xb, xd, rnd, seed=99)
        rs = host_bits(got[1])
        assert (rs[64:96, 1] == 0xFF).all() and (rs[0:32, 6] == 0xFF).all()
        a = host_bits(fq.dequantize(got[0], got[1], 32, out_dtype=torch.float32))
        b = host_bits(fq.dequantize(got[2], got[3], 32, out_dtype=torch.float32))
        fin = ~np.isnan(a)
        assert np.array_equal(np.isnan(a), np.isnan(b.T))
        assert np.array_equal(a[fin], b.T[fin])


@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_quantize_2d_ffn_weight(orc, rnd):
    w = inputs.ffn_forward()["W"]               # bf16 [2048, 5632] N(0, 0.02)
    check(orc, w, dev_bf16(w), rnd, seed=1235)
