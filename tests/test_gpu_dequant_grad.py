"""GPU parity of fp4q_dequantize (bit-exact, every code x every scale byte,
bf16 and fp32 out) and fp4q_grad_estimate (STE bit-exact; DGE within 2^-20
of the oracle's derivative, bit-exact where the clamp or the saturation
fallback sets it)."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import (assert_float_bits_equal, check_dge, dev, f64_of, host_bits,
                         to_dev_input)

pytestmark = pytest.mark.gpu


def dq_both(orc, codes, scales, block):
    want = orc.dequantize(codes, scales, block)
    cd, sd = dev(codes), dev(scales)
    for out_dtype, rnd in ((torch.bfloat16, orc.round_bf16), (torch.float32, orc.round_f32)):
        y = fq.dequantize(cd, sd, block, out_dtype)
        torch.cuda.synchronize()
        assert_float_bits_equal(host_bits(y), rnd(want), f"dequant {out_dtype} block {block}")


def test_dequant_every_code_and_scale(orc):
    rows = 256
    codes = np.zeros((rows, 16), np.uint8)
    for b in range(rows):
        c = np.arange(16, dtype=np.uint8)
        c = np.roll(c, b)
        codes[b, :8] = c[0::2] | (c[1::2] << 4)
        codes[b, 8:] = c[1::2] | (c[0::2] << 4)
    scales = np.arange(256, dtype=np.uint8).reshape(rows, 1)
    dq_both(orc, codes, scales, 32)
    dq_both(orc, codes.reshape(128, 32), scales.reshape(128, 2), 32)
    dq_both(orc, codes.reshape(512, 8), np.repeat(scales, 2).reshape(512, 1), 16)


@pytest.mark.parametrize("block", [16, 32, 64, 128])
def test_dequant_activation(orc, block):
    x = inputs.activation_sweep(rows=512, cols=2048)["X"]
    c, s = orc.quantize(x, block)
    dq_both(orc, c, s, block)
    c, s = orc.quantize(x[:3], block, round=orc.SR, seed=4)   # a ragged 3-row tensor
    dq_both(orc, c, s, block)


def test_dequant_full_activation(orc):
    d = inputs.activation_sweep()
    c, s = orc.quantize(d["X"], 32, round=orc.SR, seed=d["sr_seed"])
    dq_both(orc, c, s, 32)


# --- STE --------------------------------------------------------------------

@pytest.mark.parametrize("shape", [(4096, 2048), (3, 5), (7, 64)])
def test_ste(orc, shape):
    g = inputs.to_bf16_bits(inputs.normal(shape, 202))
    gd = to_dev_input(g)
    for out_dtype in (torch.bfloat16, torch.float32):
        o = fq.grad_estimate(fq.STE, None, gd, out_dtype=out_dtype)
        torch.cuda.synchronize()
        _, want = orc.grad_estimate(orc.STE, None, g)
        rnd = orc.round_bf16 if out_dtype == torch.bfloat16 else orc.round_f32
        assert_float_bits_equal(host_bits(o), rnd(want), f"ste {shape} {out_dtype}")
    gf = inputs.normal(shape, 203)
    o = fq.grad_estimate(fq.STE, None, to_dev_input(gf), out_dtype=torch.float32)
    assert_float_bits_equal(host_bits(o), gf, "ste f32")


# --- DGE --------------------------------------------------------------------

def dge_both(orc, x, g, block, axis, out_dtype, k=5.0, clamp=3.0, what="", ld_x=None):
    xd, gd = to_dev_input(x), to_dev_input(g)
    o = fq.grad_estimate(fq.DGE, xd, gd, block, axis, k, clamp, out_dtype=out_dtype)
    torch.cuda.synchronize()
    d_ref, _ = orc.grad_estimate(orc.DGE, x, g, block, axis, k, clamp)
    g64 = orc.bf16_to_f64(g) if g.dtype == np.uint16 else g.astype(np.float64)
    check_dge(o, d_ref, g64, orc, clamp, what)


def test_dge_tiny_ref(orc):
    d = inputs.tiny_ref()
    dge_both(orc, d["A"], d["G"], 32, fq.ROW, torch.float32, what="tiny")


@pytest.mark.parametrize("block", [16, 32, 64, 128])
def test_dge_activation_row(orc, block):
    d = inputs.activation_sweep()
    dge_both(orc, d["X"], d["G"], block, fq.ROW, torch.bfloat16, what=f"act b{block}")


@pytest.mark.parametrize("block", [16, 32, 64, 128])
def test_dge_col(orc, block):
    x = inputs.activation_sweep(rows=512, cols=1024)["X"]
    g = inputs.to_bf16_bits(inputs.normal((512, 1024), 17))
    dge_both(orc, x, g, block, fq.COL, torch.bfloat16, what=f"col b{block}")
    gf = inputs.normal((512, 1024), 18)
    dge_both(orc, x, gf, block, fq.COL, torch.float32, what=f"col f32 b{block}")
    xf = inputs.student_t((512, 1024), 19)
    dge_both(orc, xf, gf, block, fq.COL, torch.float32, what=f"col xf32 b{block}")


def test_dge_weight_gradient_shape(orc):
    """x = W bf16 [2048, 5632] with COL blocks of 32; g = an fp32 weight
    gradient of the same shape."""
    w = inputs.ffn_forward()["W"]
    g = inputs.normal(w.shape, 404, 1e-3)
    dge_both(orc, w, g, 32, fq.COL, torch.float32, what="dW")


def test_dge_ragged_cols_and_specials(orc):
    x = inputs.with_outliers(inputs.normal((64, 100), 31), 32, 30, 90.0)
    x[3, 7] = np.inf
    x[40, 50] = np.nan
    g = inputs.normal((64, 100), 33)
    dge_both(orc, x, g, 32, fq.COL, torch.float32, what="ragged col")
    dge_both(orc, x[:, :96], g[:, :96], 32, fq.ROW, torch.float32, what="row specials")


def test_dge_k1_is_ste(orc):
    d = inputs.activation_sweep(rows=256, cols=512)
    xd, gd = to_dev_input(d["X"]), to_dev_input(d["G"])
    o = fq.grad_estimate(fq.DGE, xd, gd, 32, fq.ROW, 1.0, 3.0, out_dtype=torch.bfloat16)
    assert_float_bits_equal(host_bits(o), d["G"], "k=1")
