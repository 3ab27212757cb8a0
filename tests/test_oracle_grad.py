"""Pins of the oracle's gradient estimators: STE is the identity; the DGE
staircase and its clamped derivative against closed forms, symmetry, a
finite difference of f, the clamped interval mean (by quadrature), the k = 1
special case (DGE reduces to STE) and the behaviour beyond the grid."""
import numpy as np
import pytest
from scipy import integrate

from mxfp4_block_scaled_fp4q_amd import inputs

K, CLAMP = 5.0, 3.0


def test_ste_identity(orc):
    g = inputs.to_bf16_bits(inputs.normal((16, 64), 1))
    d, out = orc.grad_estimate(orc.STE, None, g)
    assert np.all(d == 1.0)
    assert np.array_equal(orc.round_bf16(out), g)
    gf = inputs.normal((16, 64), 2)
    _, outf = orc.grad_estimate(orc.STE, None, gf)
    assert np.array_equal(orc.round_f32(outf), gf)


@pytest.mark.parametrize("delta", [0.5, 1.0, 2.0])
def test_dge_f_closed_forms(orc, delta):
    t = np.array([0.0, delta / 2, delta])
    f = orc.dge_f(t, delta, K)
    assert f[0] == 0.0 and f[1] == delta / 2 and f[2] == delta
    # monotone, and close to the staircase (step at the midpoint) for large k
    tt = np.linspace(0, delta, 1001)
    ff = orc.dge_f(tt, delta, K)
    assert np.all(np.diff(ff) >= 0)
    f50 = orc.dge_f(np.array([0.1 * delta, 0.9 * delta]), delta, 50.0)
    assert f50[0] < 0.02 * delta and f50[1] > 0.98 * delta


@pytest.mark.parametrize("delta", [0.5, 1.0, 2.0])
def test_dge_fprime_closed_forms(orc, delta):
    fp = orc.dge_fprime(np.array([0.0, delta]), delta, K, CLAMP)
    assert np.all(fp == 1.0 / K)
    # |u| = 2^-5: (1/5) * (2^-5)^(-4/5) = 0.2 * 2^4 = 3.2 -> clamped to 3.0
    u = 2.0 ** -5
    t = np.array([(1 + u) * delta / 2, (1 - u) * delta / 2, delta / 2])
    assert np.all(orc.dge_fprime(t, delta, K, CLAMP) == 3.0)
    # below u0 = (3k)^(-k/(k-1)) the clamp binds; above it does not
    u0 = (3 * K) ** (-K / (K - 1))
    assert abs(u0 - 0.0338755) < 1e-6
    t_in = (1 + u0 * 0.999) * delta / 2
    t_out = (1 + u0 * 1.001) * delta / 2
    assert orc.dge_fprime(np.array([t_in]), delta, K, CLAMP)[0] == 3.0
    assert orc.dge_fprime(np.array([t_out]), delta, K, CLAMP)[0] < 3.0
    # symmetry f'(delta - t) = f'(t)
    tt = np.random.default_rng(1).uniform(0, delta, 500)
    a = orc.dge_fprime(tt, delta, K, CLAMP)
    b = orc.dge_fprime(delta - tt, delta, K, CLAMP)
    assert np.allclose(a, b, rtol=1e-12, atol=0)


@pytest.mark.parametrize("delta", [0.5, 1.0, 2.0])
def test_dge_fprime_is_derivative_of_f(orc, delta):
    u = np.concatenate([np.linspace(-0.95, -0.06, 40), np.linspace(0.06, 0.95, 40)])
    t = (1 + u) * delta / 2
    h = 1e-6 * delta
    fd = (orc.dge_f(t + h, delta, K) - orc.dge_f(t - h, delta, K)) / (2 * h)
    fp = orc.dge_fprime(t, delta, K, 1e30)
    assert np.allclose(fd, fp, rtol=1e-5, atol=0)


def test_dge_clamped_interval_mean(orc):
    """Mean of the clamped derivative over one interval = 1 - u0^(1/k) + 3 u0
    = 0.593494 (k = 5, clamp 3); unclamped it is exactly 1 (f rises by delta)."""
    u0 = 15.0 ** (-1.25)
    closed = 1 - u0 ** (1 / K) + 3 * u0
    assert abs(closed - 0.593494) < 5e-7
    for delta in (0.5, 2.0):
        g = lambda t: orc.dge_fprime(np.array([t]), delta, K, CLAMP)[0]
        mid = delta / 2
        pts = [mid * (1 - u0), mid, mid * (1 + u0)]
        val, _ = integrate.quad(g, 0, delta, points=pts, limit=400)
        assert abs(val / delta - closed) < 1e-7
        gu = lambda t: orc.dge_fprime(np.array([t]), delta, K, 1e300)[0]
        val1, _ = integrate.quad(gu, 0, delta, points=[mid], limit=400)
        assert abs(val1 / delta - 1.0) < 1e-6


def test_dge_k1_is_ste(orc):
    x = inputs.with_outliers(inputs.normal((32, 64), 3), 4, 20, 50.0)
    g = inputs.normal((32, 64), 5)
    d, out = orc.grad_estimate(orc.DGE, x, g, 32, orc.ROW, k=1.0, clamp_max=3.0)
    assert np.all(d == 1.0)
    assert np.array_equal(orc.round_f32(out), g)


def test_dge_elementwise_table(orc):
    """Block with scale 2^0 (amax in [4, 8)): m = |x| directly."""
    m = [0.0, 0.25, 0.5, 1.0, 1.75, 2.0, 2.5, 3.0, 4.0, 5.0, 6.0, 6.5, 7.9,
         0.25 * (1 + 2 ** -5), 3.0 + 0.5 * (1 - 2 ** -5)]
    x = np.zeros((1, 32), np.float32)
    x[0, :len(m)] = m
    x[0, 20] = -5.0
    g = np.ones((1, 32), np.float32)
    g[0, 21] = -2.0
    d, out = orc.grad_estimate(orc.DGE, x, g, 32, orc.ROW, K, CLAMP)
    want = [0.2, 3.0, 0.2, 0.2, 3.0, 0.2, 3.0, 0.2, 0.2, 3.0, 0.2, 1.0, 1.0, 3.0, 3.0]
    assert np.all(d[0, :len(m)] == want)
    assert d[0, 20] == 3.0  # sign of x does not matter
    assert out[0, 21] == -2.0 * 0.2  # x = 0 there: d = 1/k
    assert np.array_equal(out, g * d)


def test_dge_col_axis_is_row_of_transpose(orc):
    x = inputs.with_outliers(inputs.normal((64, 96), 6), 7, 30, 50.0)
    g = inputs.normal((64, 96), 8)
    dc, oc = orc.grad_estimate(orc.DGE, x, g, 32, orc.COL, K, CLAMP)
    dr, orr = orc.grad_estimate(orc.DGE, np.ascontiguousarray(x.T), np.ascontiguousarray(g.T),
                                32, orc.ROW, K, CLAMP)
    assert np.array_equal(dc, dr.T) and np.array_equal(oc, orr.T)


def test_dge_nonfinite_block_is_nan(orc):
    x = np.ones((1, 64), np.float32)
    x[0, 40] = np.inf
    g = np.ones((1, 64), np.float32)
    d, _ = orc.grad_estimate(orc.DGE, x, g, 32, orc.ROW, K, CLAMP)
    assert np.all(np.isfinite(d[0, :32])) and np.all(np.isnan(d[0, 32:]))
