"""GPU parity of the on-device hot-channel choice (fp4q_hot_channels): the
per-channel fp32 errors against the oracle's float64 errors within the fp32
summation bound, the ranking exact against the library's own errors (a
deterministic sort: larger first, NaN first, ties to the lower index), and
the chosen set a valid top-n of the oracle's errors (equal to the oracle's
wherever its n-th and (n+1)-th errors are further apart than the bound)."""
import numpy as np
import pytest
import torch

import mxfp4_block_scaled_fp4q_amd as fq
from mxfp4_block_scaled_fp4q_amd import inputs
from gpu_helpers import dev_bf16, host_bits

pytestmark = pytest.mark.gpu

# fp32 squares (relative rounding 2^-24 each) summed in fp32 over at most
# 16 + 2 + rows/64 sequential additions of non-negative terms: relative error
# below (rows/64 + 20) * 2^-24, i.e. < 3e-4 for 2^17 rows.
ERR_RTOL = 3e-4


def gpu_top(err32, n):
    """The ranking rule applied to the library's own fp32 errors."""
    e = err32.astype(np.float64)
    nan = np.isnan(e)
    order = np.lexsort((np.arange(e.size), -np.where(nan, 0.0, e), ~nan))
    return np.sort(order[:n])


def check_valid_top(hot, e_ref, want, rtol=ERR_RTOL):
    """hot is a top-n of the oracle's errors e_ref up to the bound, and equals
    the oracle's own choice `want` where its ranking has a clear gap at n."""
    n = want.size
    assert hot.size == n
    if n == 0:
        return
    assert np.all(np.diff(hot) > 0) and hot[0] >= 0 and hot[-1] < e_ref.size
    nan = np.isnan(e_ref)
    sel = np.zeros(e_ref.size, bool)
    sel[hot] = True
    if nan.sum() >= n:
        assert nan[hot].all()
        return
    assert sel[nan].all(), "a NaN channel was left out"
    fin_sel = e_ref[sel & ~nan]
    rest = e_ref[~sel]
    if rest.size and fin_sel.size:
        assert fin_sel.min() >= rest.max() * (1 - 2 * rtol), "a clearly larger channel was left out"
    srt = np.sort(np.where(nan, np.inf, e_ref))[::-1]
    if n < e_ref.size and srt[n - 1] > srt[n] * (1 + 2 * rtol):
        assert hot.tolist() == want.tolist()


def run(xd, n):
    print(f"hot_channels rows={xd.shape[0]} cols={xd.shape[1]} ld={xd.stride(0)} n={n}",
          flush=True)
    hot, err = fq.hot_channels(xd, n, want_err=True)
    torch.cuda.synchronize()
    return host_bits(hot).astype(np.int64), host_bits(err)


CASES = [(1, 32, 3), (63, 96, 9), (65, 544, 49), (200, 1056, 95), (300, 2048, 184),
         (129, 5120, 461)]


@pytest.mark.parametrize("rows,cols,n", CASES)
def test_hot_channels_parity(orc, rows, cols, n):
    xf = inputs.with_outliers(inputs.normal((rows, cols), rows + cols), 7 + cols,
                              max(1, rows * cols // 200), 40.0)
    xb = inputs.to_bf16_bits(xf)
    hot, err = run(dev_bf16(xb), n)
    want, e = orc.hot_channels(xb, n)
    np.testing.assert_allclose(err, e, rtol=ERR_RTOL, atol=0)
    assert hot.tolist() == gpu_top(err, n).tolist()
    check_valid_top(hot, e, want)


def test_hot_channels_row_stride_and_edges(orc):
    rows, cols = 130, 320
    wide = inputs.to_bf16_bits(inputs.student_t((rows, cols + 64), 931))
    xd = dev_bf16(wide)[:, 64:]                      # ld = cols + 64, 128-byte offset
    xb = np.ascontiguousarray(wide[:, 64:])
    for n in (0, 1, 29, cols):
        want, e = orc.hot_channels(xb, n)
        hot, err = run(xd, n)
        np.testing.assert_allclose(err, e, rtol=ERR_RTOL, atol=0)
        assert hot.tolist() == gpu_top(err, n).tolist()
        check_valid_top(hot, e, want)
    assert run(xd, cols)[0].tolist() == list(range(cols))
    a = run(xd, 29)
    b = run(xd, 29)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1].view(np.uint32),
                                                          b[1].view(np.uint32))


def test_hot_channels_zero_ties_and_nonfinite(orc):
    x = np.zeros((70, 64), np.float32)
    hot, err = run(dev_bf16(inputs.to_bf16_bits(x)), 5)
    assert hot.tolist() == [0, 1, 2, 3, 4] and not err.any()
    x[:, 37] = 5.0                        # a tie of E2M1 rounding: error 1 per row
    x[:, 5] = -5.0
    xb = inputs.to_bf16_bits(x)
    assert run(dev_bf16(xb), 1)[0].tolist() == [5]
    hot, err = run(dev_bf16(xb), 3)
    assert hot.tolist() == [0, 5, 37] and err[5] == 70.0 and err[37] == 70.0
    xb = inputs.to_bf16_bits(inputs.normal((96, 128), 932))
    xb[50, 70] = 0x7F80                   # +inf: block 2 of row 50 is non-finite
    xb[10, 3] = 0xFFC1                    # NaN: block 0 of row 10
    hot, err = run(dev_bf16(xb), 70)
    want, e = orc.hot_channels(xb, 70)
    assert np.array_equal(np.isnan(err), np.isnan(e))
    assert np.isnan(err[:32]).all() and np.isnan(err[64:96]).all()
    assert hot.tolist() == gpu_top(err, 70).tolist()
    check_valid_top(hot, e, want)


@pytest.mark.parametrize("n", [1475, 16384])
def test_hot_channels_max_cols(orc, n):
    rows, cols = 64, 16384
    xb = inputs.to_bf16_bits(inputs.with_outliers(inputs.student_t((rows, cols), 933), 934,
                                                  4000, 20.0))
    hot, err = run(dev_bf16(xb), n)
    want, e = orc.hot_channels(xb, n)
    np.testing.assert_allclose(err, e, rtol=ERR_RTOL, atol=0)
    assert hot.tolist() == gpu_top(err, n).tolist()
    check_valid_top(hot, e, want)


def test_hot_channels_outlier_layer_full_size(orc):
    # the 13B-shaped layer (X [16384, 5120], 9% of the channels x100): the
    # planted channels are the ones chosen; sampled blocks' errors match the
    # oracle's errors of those 32-column blocks (each block's errors depend
    # on its own columns only)
    d = inputs.outlier_layer()
    xb, planted = d["X"], d["hot"]
    del d
    hot, err = run(dev_bf16(xb), planted.size)
    assert hot.tolist() == gpu_top(err, planted.size).tolist()
    assert hot.tolist() == planted.tolist()
    rng = np.random.default_rng(935)
    for b in rng.choice(xb.shape[1] // 32, size=6, replace=False):
        e = orc.channel_quant_error(np.ascontiguousarray(xb[:, b * 32:(b + 1) * 32]))
        np.testing.assert_allclose(err[b * 32:(b + 1) * 32], e, rtol=ERR_RTOL, atol=0)
