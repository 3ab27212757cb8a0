"""Pins of the oracle's random Hadamard transform before quantisation (the
backward-pass RHT of the outlier-dynamics page, sec. 4.1), whose definition
y = 2^-2.5 * H32 * D * x is computed in float64 with no evaluation order:
against scipy's Hadamard matrix; exact outputs for scaled unit vectors;
H32 H32 = 32 I; sign flips equal negated inputs; the transformed operands of
a GEMM over the transformed axis give the original product; the fp32 bound
holds for fp32 butterfly evaluations written here in two stride orders; the
validity check (rht_check) accepts every such evaluation's quantisation in
nearest-even and stochastic rounding and rejects planted mistakes (a shifted
sign mask, a missing constant, a permuted Hadamard order, the wrong random
stream, a transposed group axis); non-finite and overflowing groups; and the
quantised product over the transformed axis."""
import numpy as np
import pytest
from scipy.linalg import hadamard

from mxfp4_block_scaled_fp4q_amd import inputs


def ref_transform(x, signs):
    """float64 c * H32 * D along rows' 32-column groups, c = 2^-2.5, from
    scipy's Hadamard matrix."""
    H = hadamard(32).astype(np.float64)
    d = np.where(signs, -1.0, 1.0)
    y = np.empty(x.shape, np.float64)
    for b in range(x.shape[1] // 32):
        sl = slice(32 * b, 32 * b + 32)
        y[:, sl] = (x[:, sl].astype(np.float64) * d[sl]) @ H.T
    return y * 2.0 ** -2.5


def fp32_butterflies(xf32, signs, strides=(1, 2, 4, 8, 16), c=np.float32(2.0 ** -2.5)):
    """An fp32 evaluation of the transform along rows' groups of 32, written
    here independently of the oracle: sign flips, butterflies
    (a, b) -> (a + b, a - b) on pairs (i, i + s) for the given stride order,
    then the product by the fp32 constant."""
    v = np.where(np.asarray(signs, bool)[None, :], -xf32, xf32).astype(np.float32)
    rows, n = v.shape
    v = v.reshape(rows, n // 32, 32).copy()
    with np.errstate(over="ignore", invalid="ignore"):
        for s in strides:
            idx = np.arange(32)
            a_i = idx[(idx & s) == 0]
            a = v[:, :, a_i].copy()
            b = v[:, :, a_i + s].copy()
            v[:, :, a_i] = (a + b).astype(np.float32)
            v[:, :, a_i + s] = (a - b).astype(np.float32)
        return (v * c).astype(np.float32).reshape(rows, n)


def bf16_f32(orc, xb):
    return orc.bf16_to_f64(xb).astype(np.float32)


def test_against_scipy_hadamard(orc):
    x = inputs.student_t((16, 128), 951)
    sg = np.random.default_rng(952).random(128) < 0.5
    y, b = orc.rht_exact(x, orc.ROW, sg)
    np.testing.assert_allclose(y, ref_transform(x, sg), rtol=1e-13, atol=1e-30)
    assert np.array_equal(orc.hadamard32(), hadamard(32))
    yc, bc = orc.rht_exact(np.ascontiguousarray(x.T), orc.COL, sg)
    np.testing.assert_array_equal(yc, y.T)
    np.testing.assert_array_equal(bc, b.T)


@pytest.mark.parametrize("strides", [(1, 2, 4, 8, 16), (16, 8, 4, 2, 1), (4, 1, 16, 2, 8)])
def test_fp32_butterflies_within_bound(orc, strides):
    xb = inputs.to_bf16_bits(inputs.with_outliers(inputs.student_t((64, 256), 940), 941, 80, 60.0))
    sg = np.random.default_rng(942).random(256) < 0.5
    y, b = orc.rht_exact(xb, orc.ROW, sg)
    f = fp32_butterflies(bf16_f32(orc, xb), sg, strides).astype(np.float64)
    err = np.abs(f - y)
    assert np.all(err <= b)
    # the bound is a few rounding units, not vacuous: some errors reach a
    # fiftieth of it
    assert (err / b).max() > 0.02


def test_unit_vectors_are_exact(orc):
    H = hadamard(32)
    for j in (0, 1, 5, 17, 31):
        x = np.zeros((1, 64), np.float32)
        x[0, 32 + j] = 8.0
        sg = np.zeros(64, bool)
        sg[32 + j] = j % 2 == 1
        y, _ = orc.rht_exact(x, orc.ROW, sg)
        s = -1.0 if j % 2 else 1.0
        assert not y[0, :32].any()
        np.testing.assert_array_equal(y[0, 32:], 8.0 * s * H[:, j] * 2.0 ** -2.5)


def test_twice_is_identity(orc):
    x = inputs.normal((8, 96), 953)
    sg = np.zeros(96, bool)
    y, _ = orc.rht_exact(x, orc.ROW, sg)
    z, _ = orc.rht_exact(y.astype(np.float32), orc.ROW, sg)
    np.testing.assert_allclose(z, x, rtol=0, atol=1e-6 * np.abs(x).max())
    # H32 H32 = 32 I exactly
    H = orc.hadamard32()
    np.testing.assert_array_equal(H @ H, 32 * np.eye(32))


def test_signs_negate_inputs(orc):
    x = inputs.normal((4, 64), 954)
    sg = np.random.default_rng(955).random(64) < 0.5
    xn = np.where(sg[None, :], -x, x).astype(np.float32)
    np.testing.assert_array_equal(orc.rht_exact(x, orc.ROW, sg)[0],
                                  orc.rht_exact(xn, orc.ROW, np.zeros(64, bool))[0])


def test_gemm_over_transformed_axis_is_unchanged(orc):
    # dW = X^T dY contracts over rows: transform both along rows (COL)
    x = inputs.normal((128, 48), 956)
    g = inputs.normal((128, 40), 957)
    sg = np.random.default_rng(958).random(128) < 0.5
    tx, _ = orc.rht_exact(x, orc.COL, sg)
    tg, _ = orc.rht_exact(g, orc.COL, sg)
    exact = x.astype(np.float64).T @ g.astype(np.float64)
    np.testing.assert_allclose(tx.T @ tg, exact, rtol=0, atol=1e-12 * np.abs(exact).max())


def test_nonfinite_and_overflowing_groups(orc):
    xb = inputs.to_bf16_bits(inputs.normal((4, 96), 959))
    xb[1, 40] = 0x7F80            # +inf: group 1 of row 1
    xb[3, 70] = 0x7F7F            # two of the largest finite bf16 in one group:
    xb[3, 71] = 0x7F7F            # every fp32 evaluation overflows
    sg = np.zeros(96, bool)
    codes, scales = orc.rht_quantize(xb, orc.ROW, sg)
    assert scales[1, 1] == 0xFF and (codes[1, 16:32] == 0).all()
    assert scales[3, 2] == 0xFF and (codes[3, 32:48] == 0).all()
    assert (scales[[0, 2]] != 0xFF).all() and scales[1, 0] != 0xFF and scales[3, 0] != 0xFF
    r = orc.rht_check(xb, orc.ROW, sg, codes, scales)
    assert r["bad_scales"] == 0 and r["bad_codes"] == 0, r
    # those groups may not come back with a finite scale
    bad = scales.copy()
    bad[3, 2] = 130
    assert orc.rht_check(xb, orc.ROW, sg, codes, bad)["bad_scales"] == 1
    # and a finite group may not come back as 0xFF
    bad = scales.copy()
    bad[0, 0] = 0xFF
    assert orc.rht_check(xb, orc.ROW, sg, codes, bad)["bad_scales"] == 1


def _operand(orc, shape, seed):
    return inputs.to_bf16_bits(inputs.with_outliers(inputs.student_t(shape, seed), seed + 1,
                                                    max(1, shape[0] * shape[1] // 250), 40.0))


@pytest.mark.parametrize("rnd", ["rne", "sr"])
@pytest.mark.parametrize("axis", ["row", "col"])
def test_check_accepts_fp32_evaluations(orc, axis, rnd):
    """The nominal quantisation and quantisations of fp32 butterfly
    evaluations in two stride orders all pass the check; most elements are
    fixed uniquely by the bound."""
    ax = orc.ROW if axis == "row" else orc.COL
    r = orc.RNE if rnd == "rne" else orc.SR
    xb = _operand(orc, (96, 160), 943)
    n = 160 if axis == "row" else 96
    sg = np.random.default_rng(944).random(n) < 0.5
    res = orc.rht_check(xb, ax, sg, *orc.rht_quantize(xb, ax, sg, r, 77, 5), round=r, seed=77,
                        rng_offset=5)
    assert res["bad_scales"] == 0 and res["bad_codes"] == 0, res
    assert res["exact_elems"] > 0.99 * res["elems"], res
    xf = bf16_f32(orc, xb)
    for strides in ((1, 2, 4, 8, 16), (16, 8, 4, 2, 1)):
        if axis == "row":
            f = fp32_butterflies(xf, sg, strides)
        else:
            f = np.ascontiguousarray(fp32_butterflies(np.ascontiguousarray(xf.T), sg, strides).T)
        q = orc.quantize(f, 32, ax, r, 77, 5)
        res = orc.rht_check(xb, ax, sg, *q, round=r, seed=77, rng_offset=5)
        assert res["bad_scales"] == 0 and res["bad_codes"] == 0, (strides, res)


@pytest.mark.parametrize("rnd", ["rne", "sr"])
def test_check_rejects_planted_mistakes(orc, rnd):
    r = orc.RNE if rnd == "rne" else orc.SR
    xb = _operand(orc, (64, 128), 945)
    xf = bf16_f32(orc, xb)
    sg = np.random.default_rng(946).random(128) < 0.5

    def check(f, seed=11, off=0):
        q = orc.quantize(f, 32, orc.ROW, r, seed, off)
        res = orc.rht_check(xb, orc.ROW, sg, *q, round=r, seed=11, rng_offset=0)
        return res["bad_scales"] + res["bad_codes"]

    assert check(fp32_butterflies(xf, sg)) == 0
    # the sign mask shifted by one position
    assert check(fp32_butterflies(xf, np.roll(sg, 1))) > 100
    # the constant left out (values 4 sqrt 2 too large)
    assert check(fp32_butterflies(xf, sg, c=np.float32(1.0))) > 100
    # a Hadamard matrix in another row order: outputs permuted within groups
    f = fp32_butterflies(xf, sg).reshape(64, 4, 32)[:, :, ::-1].reshape(64, 128)
    assert check(np.ascontiguousarray(f)) > 100
    # groups taken down the columns instead of along the rows
    # (the first 64 x 64 square transformed along its columns)
    f = fp32_butterflies(xf, sg).copy()
    f[:, :64] = fp32_butterflies(np.ascontiguousarray(xf[:, :64].T), sg[:64]).T
    assert check(f) > 100
    if r == orc.SR:
        # another random stream, and the counters shifted by one
        assert check(fp32_butterflies(xf, sg), seed=12) > 100
        assert check(fp32_butterflies(xf, sg), off=1) > 100


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
