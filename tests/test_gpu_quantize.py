"""GPU parity of fp4q_quantize against the CPU oracle: codes and E8M0 bytes
bit-exact for RNE and stochastic rounding, ROW and COL blocks, bf16 and fp32
inputs, every block size, strided rows, ragged shapes, offsets, special
values, and the full-size tensors of the layer workloads."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import assert_same_bits, host_bits, to_dev_input

pytestmark = pytest.mark.gpu


def run_both(orc, x, block, axis=fq.ROW, rnd=fq.RNE, seed=0, off=0, ld_pad=0):
    xd = to_dev_input(x)
    if ld_pad:
        big = torch.zeros((x.shape[0], x.shape[1] + ld_pad), dtype=xd.dtype, device="cuda")
        big[:, :x.shape[1]] = xd
        xd = big[:, :x.shape[1]]
    c, s = fq.quantize(xd, block, axis, rnd, seed, off)
    torch.cuda.synchronize()
    co, so = orc.quantize(x, block, axis, rnd, seed, off)
    what = f"shape={x.shape} block={block} axis={axis} round={rnd} seed={seed} off={off}"
    assert_same_bits(host_bits(s), so, "scales " + what)
    assert_same_bits(host_bits(c), co, "codes " + what)


def test_tiny_ref(orc):
    d = inputs.tiny_ref()
    for name in ("A", "B"):
        run_both(orc, d[name], 32)
        run_both(orc, d[name], 32, fq.COL)
        run_both(orc, d[name], 32, rnd=fq.SR, seed=7)


@pytest.mark.parametrize("block", [16, 32, 64, 128])
@pytest.mark.parametrize("rnd", [fq.RNE, fq.SR])
def test_activation_sweep_row(orc, block, rnd):
    d = inputs.activation_sweep()
    run_both(orc, d["X"], block, fq.ROW, rnd, d["sr_seed"])


@pytest.mark.parametrize("block", [16, 32, 64, 128])
def test_activation_col(orc, block):
    x = inputs.activation_sweep(rows=1024, cols=1536)["X"]
    run_both(orc, x, block, fq.COL, fq.RNE)
    run_both(orc, x, block, fq.COL, fq.SR, 1234)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("axis", [fq.ROW, fq.COL])
@pytest.mark.parametrize("rnd", [fq.RNE, fq.SR])
def test_ragged_and_offsets(orc, dtype, axis, rnd):
    # rows / cols that leave partial waves, partial column groups (COL) and
    # SR offsets that straddle Philox counters
    cols = 203 if axis == fq.COL else 192
    pad = (8 - cols % 8) % 8  # keeps the row stride 16-byte aligned
    x = inputs.with_outliers(inputs.normal((96, cols), 5), 6, 40, 80.0)
    if dtype == "bf16":
        x = inputs.to_bf16_bits(x)
    for off in (0, 5, 8 * 1001 + 3):
        run_both(orc, x, 32, axis, rnd, 99, off, ld_pad=pad)
    run_both(orc, x, 16, axis, rnd, 99, 1, ld_pad=pad)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
def test_col_aligned_edges(orc, dtype):
    """COL pass with columns a multiple of 8 (unconditional loads; lanes
    wholly outside the matrix read its first rows and columns, which reach no
    stored output): partial row and column tiles, 32-bit tile offsets, and
    columns that are not a multiple of 8 (element loads at the edge)."""
    x = inputs.with_outliers(inputs.normal((640, 1192), 61), 12, 60, 90.0)
    if dtype == "bf16":
        x = inputs.to_bf16_bits(x)
    run_both(orc, x, 32, fq.COL, fq.RNE)
    run_both(orc, x, 16, fq.COL, fq.SR, 77)
    run_both(orc, x, 64, fq.COL, fq.SR, 78, 8 * 55, ld_pad=8)
    run_both(orc, x, 32, fq.COL, fq.SR, 79, 3)
    run_both(orc, x[:, :1190], 32, fq.COL, fq.RNE, ld_pad=2)
    run_both(orc, x[:, :1190], 32, fq.COL, fq.SR, 80, ld_pad=2)


def test_col_huge_row_stride(orc):
    """A row stride so long that a column tile's extent reaches 2^31 bytes:
    the host takes the element-load form (64-bit addressing) instead of the
    32-bit tile offsets; results are the same bits."""
    x = inputs.to_bf16_bits(inputs.with_outliers(inputs.normal((64, 1024), 81), 9, 40, 60.0))
    ld = 8_500_000  # 128 rows x ld x 2 bytes > 2^31
    big = torch.zeros((64, ld), dtype=torch.bfloat16, device="cuda")
    big[:, :1024] = to_dev_input(x)
    xd = big[:, :1024]
    for rnd, seed in ((fq.RNE, 0), (fq.SR, 5)):
        c, s_ = fq.quantize(xd, 32, fq.COL, rnd, seed)
        (rc, rs), (cc, cs) = fq.quantize_dual(xd, 32, rnd, seed, rnd, seed)
        torch.cuda.synchronize()
        co, so = orc.quantize(x, 32, fq.COL, rnd, seed)
        ro, rso = orc.quantize(x, 32, fq.ROW, rnd, seed)
        what = f"ld={ld} round={rnd}"
        assert_same_bits(host_bits(s_), so, "col scales " + what)
        assert_same_bits(host_bits(c), co, "col codes " + what)
        assert_same_bits(host_bits(cs), so, "dual col scales " + what)
        assert_same_bits(host_bits(cc), co, "dual col codes " + what)
        assert_same_bits(host_bits(rs), rso, "dual row scales " + what)
        assert_same_bits(host_bits(rc), ro, "dual row codes " + what)
    del big


@pytest.mark.parametrize("axis", [fq.ROW, fq.COL])
def test_strided_rows(orc, axis):
    x = inputs.to_bf16_bits(inputs.normal((64, 256), 8))
    run_both(orc, x, 32, axis, fq.RNE, ld_pad=8)
    run_both(orc, x, 32, axis, fq.SR, 3, ld_pad=24)
    xf = inputs.normal((64, 256), 9)
    run_both(orc, xf, 64, axis, fq.SR, 4, ld_pad=4)


@pytest.mark.parametrize("block", [16, 32, 128])
def test_every_bf16_pattern(orc, block):
    """All 65536 bf16 bit patterns (NaN and Inf blocks included), in two
    orders so each value meets different block maxima."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(block)
    for arr in (bits, rng.permutation(bits)):
        x = arr.reshape(-1, 256)
        run_both(orc, x, block, fq.ROW, fq.RNE)
        run_both(orc, x, block, fq.ROW, fq.SR, 11)
        run_both(orc, x, block, fq.COL, fq.RNE)
        run_both(orc, x, block, fq.COL, fq.SR, 12)


def test_fp32_special_values(orc):
    """Random fp32 bit patterns (subnormals, NaN, Inf included), plus blocks
    whose elements sit far below the block maximum (scaled values in the
    subnormal range, where the truncated 16-bit fraction is 0 and SR keeps
    the lower neighbour)."""
    rng = np.random.default_rng(21)
    bits = rng.integers(0, 1 << 32, (128, 256), dtype=np.uint64).astype(np.uint32)
    x = bits.view(np.float32).copy()
    for block in (16, 32):
        run_both(orc, x, block, fq.ROW, fq.RNE)
        run_both(orc, x, block, fq.ROW, fq.SR, 5)
        run_both(orc, x, block, fq.COL, fq.RNE)
        run_both(orc, x, block, fq.COL, fq.SR, 6)
    y = np.zeros((64, 32), np.float32)
    y[:, 0] = 3.0e38
    y[:, 1:] = rng.uniform(-1, 1, (64, 31)).astype(np.float32) * np.float32(1e-38)
    y[::2, 2] = np.float32(1e-45)
    y[1::2, 3] = -np.float32(1e-45)
    run_both(orc, y, 32, fq.ROW, fq.RNE)
    for seed in range(4):
        run_both(orc, y, 32, fq.ROW, fq.SR, seed)


def test_ffn_forward_operands(orc):
    d = inputs.ffn_forward()
    run_both(orc, d["X"], 32, fq.ROW)
    run_both(orc, d["W"], 32, fq.COL)


def test_ffn_backward_operands(orc):
    d = inputs.ffn_backward_grad()
    run_both(orc, d["dY"], 32, fq.ROW, fq.SR, d["seed_row"])
    run_both(orc, d["dY"], 32, fq.COL, fq.SR, d["seed_col"])
    f = inputs.ffn_forward()
    run_both(orc, f["X"], 32, fq.COL)
    run_both(orc, f["W"], 32, fq.ROW)


def test_outlier_layer_operands(orc):
    d = inputs.outlier_layer()
    run_both(orc, d["X"], 32, fq.ROW)
    run_both(orc, d["W"], 32, fq.COL)


@pytest.mark.parametrize("dtype", ["bf16", "f32"])
@pytest.mark.parametrize("rnd", [fq.RNE, fq.SR])
def test_row_partial_waves(orc, dtype, rnd):
    """Dense ROW inputs whose 8-element chunk count leaves a partial wave
    (and a single chunk): the loads past the last chunk are clamped and
    their lanes write nothing."""
    for shape, block in (((1, 16), 16), ((5, 48), 16), ((3, 96), 32), ((7, 128), 64),
                         ((2, 128), 128)):
        x = inputs.with_outliers(inputs.normal(shape, 31), 32, 1, 40.0)
        if dtype == "bf16":
            x = inputs.to_bf16_bits(x)
        run_both(orc, x, block, fq.ROW, rnd, 77)
