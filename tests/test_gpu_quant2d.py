"""GPU parity of the two-dimensional block scaling (fp4q_quantize_2d with
32 x 32 squares, fp4q_quantize_2d_tile with 16 x 16): codes and scales in
both layouts bit for bit against the oracle, nearest-even and stochastic,
over ragged region counts, a padded row stride, non-finite squares and the
LLaMA-1B FFN weight shape; the two layouts dequantise to one matrix and its
transpose."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import assert_same_bits, dev_bf16, host_bits

pytestmark = pytest.mark.gpu

NAMES = ("row_codes", "row_scales", "col_codes", "col_scales")


def check(orc, xb, xd, rnd, seed=0, off=0, tile=32):
    print(f"quantize_2d tile={tile} shape={xb.shape} ld={xd.stride(0)} round={rnd} seed={seed} "
          f"off={off}", flush=True)
    r = fq.RNE if rnd == "rne" else fq.SR
    got = fq.quantize_2d(xd, r, seed, off, tile=tile)
    torch.cuda.synchronize()
    want = orc.quantize_2d(xb, tile, orc.RNE if rnd == "rne" else orc.SR, seed, off)
    for n, g, w in zip(NAMES, got, want):
        assert_same_bits(host_bits(g), w, n)
    return got


@pytest.mark.parametrize("tile", [32, 16])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("shape", [(32, 32), (96, 160), (128, 128), (288, 416), (160, 4128)])
def test_quantize_2d_parity(orc, rnd, shape, tile):
    xb = inputs.to_bf16_bits(inputs.with_outliers(inputs.student_t(shape, sum(shape)), 5,
                                                  max(1, shape[0] * shape[1] // 300), 30.0))
    check(orc, xb, dev_bf16(xb), rnd, seed=1234 + shape[1], off=7 * shape[0], tile=tile)


@pytest.mark.parametrize("tile", [32, 16])
def test_quantize_2d_row_stride_nonfinite_and_one_matrix(orc, tile):
    wide = inputs.to_bf16_bits(inputs.normal((192, 256 + 96), 941))
    wide[70, 96 + 40] = 0x7F80        # +inf: square (2, 1) of the view
    wide[5, 96 + 200] = 0xFFC0        # NaN: square (0, 6)
    xd = dev_bf16(wide)[:, 96:]
    xb = np.ascontiguousarray(wide[:, 96:])
    t = tile
    for rnd in ("rne", "sr"):
        got = check(orc, xb, xd, rnd, seed=99, tile=t)
        rs = host_bits(got[1])
        r_inf, c_inf = 70 // t, 40 // t
        r_nan, c_nan = 5 // t, 200 // t
        assert (rs[t * r_inf:t * r_inf + t, c_inf] == 0xFF).all()
        assert (rs[t * r_nan:t * r_nan + t, c_nan] == 0xFF).all()
        assert (rs == 0xFF).sum() == 2 * t
        a = host_bits(fq.dequantize(got[0], got[1], t, out_dtype=torch.float32))
        b = host_bits(fq.dequantize(got[2], got[3], t, out_dtype=torch.float32))
        fin = ~np.isnan(a)
        assert np.array_equal(np.isnan(a), np.isnan(b.T))
        assert np.array_equal(a[fin], b.T[fin])


@pytest.mark.parametrize("tile", [32, 16])
@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_quantize_2d_ffn_weight(orc, rnd, tile):
    w = inputs.ffn_forward()["W"]               # bf16 [2048, 5632] N(0, 0.02)
    check(orc, w, dev_bf16(w), rnd, seed=1235, tile=tile)
