"""Pins of the oracle's random Hadamard transform before quantisation (the
backward-pass RHT of the outlier-dynamics page, sec. 4.1): the fp32 transform
against scipy's Hadamard matrix in float64 within the fp32 rounding bound;
exact outputs for scaled unit vectors; H32 H32 = 32 I (applying it twice
returns the input up to rounding); sign flips equal negated inputs; the
transformed operands of a GEMM over the transformed axis give the original
product; non-finite groups; and the quantised product over the transformed
axis, which stays as accurate as the plain quantised product only when both
operands share the transform."""
import numpy as np
import pytest
from scipy.linalg import hadamard

from mxfp4_block_scaled_fp4q_amd import inputs


def ref_transform(x, signs):
    """float64 c * H32 * D along rows' 32-column groups, c = 2^-2.5."""
    H = hadamard(32).astype(np.float64)
    d = np.where(signs, -1.0, 1.0)
    y = np.empty(x.shape, np.float64)
    for b in range(x.shape[1] // 32):
        sl = slice(32 * b, 32 * b + 32)
        y[:, sl] = (x[:, sl].astype(np.float64) * d[sl]) @ H.T
    return y * 2.0 ** -2.5


def test_against_scipy_hadamard(orc):
    x = inputs.student_t((16, 128), 951)
    sg = np.random.default_rng(952).random(128) < 0.5
    y = orc.rht_transform(x, orc.ROW, sg)
    ref = ref_transform(x, sg)
    # 5 rounded additions and one product, each relative 2^-24 of partial sums
    bound = 8 * 2.0 ** -24 * (np.abs(x).reshape(16, 4, 32).sum(axis=2).repeat(32, axis=1) * 2 ** -2.5)
    assert np.all(np.abs(y - ref) <= bound)
    yc = orc.rht_transform(np.ascontiguousarray(x.T), orc.COL, sg)
    np.testing.assert_array_equal(yc, y.T)


def test_unit_vectors_are_exact(orc):
    H = hadamard(32)
    c = float(orc.RHT_C)
    for j in (0, 1, 5, 17, 31):
        x = np.zeros((1, 64), np.float32)
        x[0, 32 + j] = 8.0
        sg = np.zeros(64, bool)
        sg[32 + j] = j % 2 == 1
        y = orc.rht_transform(x, orc.ROW, sg)
        s = -1.0 if j % 2 else 1.0
        assert not y[0, :32].any()
        np.testing.assert_array_equal(y[0, 32:], (8.0 * s * H[:, j] * c).astype(np.float32))


def test_twice_is_identity_up_to_rounding(orc):
    x = inputs.normal((8, 96), 953)
    sg = np.zeros(96, bool)
    y = orc.rht_transform(orc.rht_transform(x, orc.ROW, sg), orc.ROW, sg)
    np.testing.assert_allclose(y, x, rtol=0, atol=1e-5 * np.abs(x).max())


def test_signs_negate_inputs(orc):
    x = inputs.normal((4, 64), 954)
    sg = np.random.default_rng(955).random(64) < 0.5
    xn = np.where(sg[None, :], -x, x).astype(np.float32)
    np.testing.assert_array_equal(orc.rht_transform(x, orc.ROW, sg),
                                  orc.rht_transform(xn, orc.ROW, np.zeros(64, bool)))


def test_gemm_over_transformed_axis_is_unchanged(orc):
    # dW = X^T dY contracts over rows: transform both along rows (COL)
    x = inputs.normal((128, 48), 956)
    g = inputs.normal((128, 40), 957)
    sg = np.random.default_rng(958).random(128) < 0.5
    tx = orc.rht_transform(x, orc.COL, sg).astype(np.float64)
    tg = orc.rht_transform(g, orc.COL, sg).astype(np.float64)
    exact = x.astype(np.float64).T @ g.astype(np.float64)
    np.testing.assert_allclose(tx.T @ tg, exact, rtol=0, atol=1e-5 * np.abs(exact).max())


def test_nonfinite_group(orc):
    xb = inputs.to_bf16_bits(inputs.normal((4, 64), 959))
    xb[1, 40] = 0x7F80
    codes, scales = orc.rht_quantize(xb, orc.ROW, np.zeros(64, bool))
    assert scales[1, 1] == 0xFF and (codes[1, 16:] == 0).all()
    assert (scales[[0, 2, 3]] != 0xFF).all() and scales[1, 0] != 0xFF


@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_quantised_product_over_transformed_axis(orc, rnd):
    # the product of the quantised transformed operands stays as close to the
    # exact product as the plain quantised product (within 25%); operands
    # transformed with different signs (a transform not shared by both
    # sides of the contraction) are far off
    m, k, n = 512, 64, 64
    x = inputs.with_outliers(inputs.student_t((m, k), 960), 961, 40, 30.0)
    g = inputs.with_outliers(inputs.student_t((m, n), 962), 963, 40, 30.0)
    xb, gb = inputs.to_bf16_bits(x), inputs.to_bf16_bits(g)
    exact = orc.bf16_to_f64(xb).T @ orc.bf16_to_f64(gb)
    r = orc.RNE if rnd == "rne" else orc.SR
    rng = np.random.default_rng(964)
    sg, sg2 = rng.random(m) < 0.5, rng.random(m) < 0.5

    def prod(qa, qb):
        return orc.dequantize(*qa, 32) @ orc.dequantize(*qb, 32).T

    plain = prod(orc.quantize(xb, 32, orc.COL, r, 5), orc.quantize(gb, 32, orc.COL, r, 6))
    rot = prod(orc.rht_quantize(xb, orc.COL, sg, r, 5), orc.rht_quantize(gb, orc.COL, sg, r, 6))
    bad = prod(orc.rht_quantize(xb, orc.COL, sg, r, 5), orc.rht_quantize(gb, orc.COL, sg2, r, 6))
    e_plain, e_rot, e_bad = (np.linalg.norm(p - exact) for p in (plain, rot, bad))
    assert e_rot < 1.25 * e_plain, (e_rot, e_plain)
    assert e_bad > 0.5 * np.linalg.norm(exact), (e_bad, np.linalg.norm(exact))
