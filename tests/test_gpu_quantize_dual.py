"""GPU parity of fp4q_quantize_dual (both block orientations of one tensor
in one pass) against the CPU oracle's two separate quantisations: codes and
E8M0 bytes bit-exact for every rounding pair, block size, ragged tiles,
strided rows, SR offsets that straddle Philox counters, every bf16 bit
pattern, fp32 input, and the full-size backward gradient of the layer
workload."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import assert_same_bits, host_bits, to_dev_input

pytestmark = pytest.mark.gpu


def run_dual(orc, x, block, rr=fq.RNE, sr_row=0, rc=fq.RNE, sr_col=0, off=0, ld_pad=0):
    xd = to_dev_input(x)
    if ld_pad:
        big = torch.zeros((x.shape[0], x.shape[1] + ld_pad), dtype=xd.dtype, device="cuda")
        big[:, :x.shape[1]] = xd
        xd = big[:, :x.shape[1]]
    (rcodes, rscales), (ccodes, cscales) = fq.quantize_dual(xd, block, rr, sr_row, rc, sr_col, off)
    torch.cuda.synchronize()
    what = (f"shape={x.shape} block={block} rounds=({rr},{rc}) seeds=({sr_row},{sr_col}) "
            f"off={off}")
    co, so = orc.quantize(x, block, fq.ROW, rr, sr_row, off)
    assert_same_bits(host_bits(rscales), so, "row scales " + what)
    assert_same_bits(host_bits(rcodes), co, "row codes " + what)
    co, so = orc.quantize(x, block, fq.COL, rc, sr_col, off)
    assert_same_bits(host_bits(cscales), so, "col scales " + what)
    assert_same_bits(host_bits(ccodes), co, "col codes " + what)


@pytest.mark.parametrize("block", [16, 32, 64, 128])
@pytest.mark.parametrize("rounds", [(fq.RNE, fq.RNE), (fq.SR, fq.SR), (fq.SR, fq.RNE),
                                    (fq.RNE, fq.SR)])
def test_dual_activation(orc, block, rounds):
    x = inputs.activation_sweep(rows=512, cols=1536)["X"]
    run_dual(orc, x, block, rounds[0], 1234, rounds[1], 1235)


@pytest.mark.parametrize("block", [16, 32, 64, 128])
def test_dual_shared_random_stream(orc, block):
    """Equal seeds: both orientations draw from one stream (one Philox call
    per row of 8 columns serves both)."""
    x = inputs.activation_sweep(rows=512, cols=1536)["X"]
    run_dual(orc, x, block, fq.SR, 1234, fq.SR, 1234)
    y = inputs.to_bf16_bits(inputs.with_outliers(inputs.normal((320, 416), 33), 32, 60, 90.0))
    for off in (0, 5, 8 * 777 + 3):
        run_dual(orc, y, 32, fq.SR, 99, fq.SR, 99, off)


@pytest.mark.parametrize("rounds", [(fq.RNE, fq.RNE), (fq.SR, fq.SR)])
def test_dual_ragged_tiles_and_offsets(orc, rounds):
    # 320 rows: a partial 256-row tile; 416 columns: a partial 128-column tile
    x = inputs.to_bf16_bits(inputs.with_outliers(inputs.normal((320, 416), 31), 32, 60, 90.0))
    for off in (0, 5, 8 * 777 + 3):
        run_dual(orc, x, 32, rounds[0], 7, rounds[1], 8, off)
    run_dual(orc, x, 16, rounds[0], 9, rounds[1], 10, 1)


def test_dual_aligned_edges(orc):
    """640 x 1184 is 5 x 10 tiles of 128 x 128 with a partial last column
    tile: lanes wholly outside the matrix read its first rows and columns,
    which reach no stored output; offsets 5 (not a multiple of 8) take the
    element-load form."""
    x = inputs.to_bf16_bits(inputs.with_outliers(inputs.normal((640, 1184), 51), 32, 60, 90.0))
    run_dual(orc, x, 32, fq.RNE, 0, fq.RNE, 0)
    run_dual(orc, x, 32, fq.SR, 7, fq.SR, 7)
    run_dual(orc, x, 16, fq.SR, 7, fq.SR, 8, 16)
    run_dual(orc, x, 32, fq.RNE, 0, fq.SR, 9, 5)
    run_dual(orc, x, 32, fq.SR, 10, fq.RNE, 0, ld_pad=8)


def test_dual_strided_rows_and_fp32(orc):
    x = inputs.to_bf16_bits(inputs.normal((128, 256), 41))
    run_dual(orc, x, 32, fq.SR, 3, fq.SR, 4, ld_pad=8)
    xf = inputs.normal((64, 256), 42)
    run_dual(orc, xf, 32, fq.RNE, 0, fq.SR, 5)
    run_dual(orc, xf, 64, fq.SR, 6, fq.RNE, 0, ld_pad=4)


@pytest.mark.parametrize("block", [16, 32, 128])
def test_dual_every_bf16_pattern(orc, block):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rng = np.random.default_rng(block + 100)
    for arr in (bits, rng.permutation(bits)):
        x = arr.reshape(-1, 256)
        run_dual(orc, x, block, fq.RNE, 0, fq.RNE, 0)
        run_dual(orc, x, block, fq.SR, 11, fq.SR, 12)


def test_dual_ffn_backward_gradient(orc):
    d = inputs.ffn_backward_grad()
    run_dual(orc, d["dY"], 32, fq.SR, d["seed_row"], fq.SR, d["seed_col"])
    run_dual(orc, d["dY"], 32, fq.SR, d["seed_row"], fq.SR, d["seed_row"])


def test_dual_matches_separate_calls():
    """Same device, same inputs: the fused pass equals two quantize calls."""
    f = inputs.ffn_forward()
    for name in ("X", "W"):
        xd = to_dev_input(f[name])
        (rc, rs), (cc, cs) = fq.quantize_dual(xd, 32)
        rc2, rs2 = fq.quantize(xd, 32, fq.ROW)
        cc2, cs2 = fq.quantize(xd, 32, fq.COL)
        torch.cuda.synchronize()
        for a, b in ((rc, rc2), (rs, rs2), (cc, cc2), (cs, cs2)):
            assert torch.equal(a, b), name
