"""Pins of the oracle's state codec (layout 0: key-row smoothing + symmetric
value-column INT8 scales) and of the DAMP split (fp16 rows + column-only
INT8 rows).

Sources: LeapQuant project page, residual-smoothing paragraph (rows are
balanced before quantization); STEPQuant page (key-row and value-column
scales); DAMP abstract (high-risk channels at higher precision, the rest in
INT8); LinQuant Figure 7 caption (per-channel scales absorb a consistent
diagonal rescaling).

The pins are invariants, closed forms, hand-derived small examples and an
exhaustive search over all 255 codes; none retypes the codec's loop.
"""
import numpy as np
import pytest

import synth


def _states(seed, nh=4, dk=16, dv=24, scale=1.0):
    X = synth.random_states(seed, nh, dk, dv, scale)
    g = synth.misc_rng(seed, 9)
    # make magnitudes uneven along both axes, as the pages describe
    X *= (2.0 ** g.uniform(-6, 6, (nh, dk, 1))).astype(np.float32)
    X *= (2.0 ** g.uniform(-3, 3, (nh, 1, dv))).astype(np.float32)
    return X


def test_hand_worked_example(orc):
    # Rows [4, y]: row max 4 -> s = 2, rho = 1/2 exactly, so Y = [2, y/2].
    # Column 0: m = 2, iota = 63.5, every t = 127.
    # Column 1: m = 127/64 -> iota = 64 exactly and c = 1/64 exactly;
    # t = 64 * y/2 gives 127, 2.5 (tie -> 2), 3.5 (tie -> 4), -2.5 (-> -2).
    X = np.array([[[4.0, 2 * 127 / 64], [4.0, 2 * 5 / 128], [4.0, 2 * 7 / 128],
                   [4.0, -2 * 5 / 128]]], np.float32)
    Q, s, c = orc.quantize(X)
    assert Q[0].tolist() == [[127, 127], [127, 2], [127, 4], [127, -2]]
    assert s[0].tolist() == [2.0, 2.0, 2.0, 2.0]
    assert c[0, 1] == np.float32(1 / 64)
    assert c[0, 0] == np.float32(np.float32(2.0) / np.float32(127.0))


def test_rounding_takes_the_exact_product(orc):
    # Rows [4, x]: s = 2 and rho = 1/2 exactly, so Y = x/2.  Column 1 has
    # m = 1.5, iota = fp32(127/1.5) = 84.66666412353516.  For these Y the
    # exact product Y * iota lies just off a half-integer while its fp32
    # rounding lands on it: 0.50000002 -> 1, 7.49999998 -> 7, 8.50000011 -> 9
    # (rounding the fp32 product instead would give 0, 8, 8).
    ys = [0.0059055122546851635, 0.08858267962932587, 0.10039370507001877]
    X = np.array([[[4.0, 3.0]] + [[4.0, 2 * y] for y in ys]], np.float32)
    Q, s, c = orc.quantize(X)
    assert Q[0].tolist() == [[127, 127], [127, 1], [127, 7], [127, 9]]


def test_code_range_and_full_scale(orc):
    X = _states(11)
    Q, s, c = orc.quantize(X)
    assert Q.min() >= -127 and Q.max() <= 127
    # every non-zero column reaches full scale
    assert np.all(np.abs(Q).max(axis=1) == 127)


def test_reconstruction_bound(orc):
    X = _states(12, nh=6)
    Q, s, c = orc.quantize(X)
    D = orc.dequantize(Q, s, c).astype(np.float64)
    err = np.abs(D - X)
    bound = s[:, :, None].astype(np.float64) * c[:, None, :] * (0.5 + 2.0 ** -10)
    assert np.all(err <= bound + np.abs(X) * 2.0 ** -22)
    # and the bound is tight: some error is near half a step
    assert np.max(err / bound) > 0.45


def test_sign_symmetry(orc):
    X = _states(13)
    Q1, s1, c1 = orc.quantize(X)
    Q2, s2, c2 = orc.quantize(-X)
    assert np.array_equal(Q2, -Q1) and np.array_equal(s1, s2) and np.array_equal(c1, c2)


@pytest.mark.parametrize("m", [-3, -1, 1, 2, 5])
def test_power_of_four_scaling(orc, m):
    X = _states(14)
    Q1, s1, c1 = orc.quantize(X)
    Q2, s2, c2 = orc.quantize(X * np.float32(4.0 ** m))
    assert np.array_equal(Q1, Q2)
    assert np.array_equal(s2, s1 * np.float32(2.0 ** m))
    assert np.array_equal(c2, c1 * np.float32(2.0 ** m))


def test_smoothing_scale_is_sqrt_of_row_max(orc):
    # The smoothing scale of key row i squares back to the row's largest
    # magnitude, so smoothing halves every row's dynamic range in log scale;
    # scaling one row by 4^m scales only that row's scale, by exactly 2^m.
    X = _states(15)
    Q1, s1, c1 = orc.quantize(X)
    rmax = np.abs(X).max(axis=2).astype(np.float64)
    np.testing.assert_allclose(s1.astype(np.float64) ** 2, rmax, rtol=2.0 ** -22)
    g = synth.misc_rng(15, 1)
    m = g.integers(-4, 5, (X.shape[0], X.shape[1], 1))
    Q2, s2, c2 = orc.quantize(X * (4.0 ** m).astype(np.float32))
    assert np.array_equal(s2, s1 * (2.0 ** m[..., 0]).astype(np.float32))


def test_permutations_commute(orc):
    X = _states(16)
    g = synth.misc_rng(16, 1)
    pr = g.permutation(X.shape[1])
    pc = g.permutation(X.shape[2])
    Q1, s1, c1 = orc.quantize(X)
    Q2, s2, c2 = orc.quantize(np.ascontiguousarray(X[:, pr][:, :, pc]))
    assert np.array_equal(Q2, Q1[:, pr][:, :, pc])
    assert np.array_equal(s2, s1[:, pr]) and np.array_equal(c2, c1[:, pc])


def test_zero_rows_and_columns(orc):
    X = _states(17)
    X[:, 3, :] = 0
    X[:, :, 5] = 0
    X[1] = 0
    Q, s, c = orc.quantize(X)
    assert np.all(Q[:, 3, :] == 0) and np.all(s[:, 3] == 0)
    assert np.all(Q[:, :, 5] == 0) and np.all(c[:, 5] == 0)
    assert np.all(Q[1] == 0) and np.all(s[1] == 0) and np.all(c[1] == 0)


def test_denormal_inputs_are_kept(orc):
    # A tile made only of subnormals is coded like any other (no flush to
    # zero): scales are non-zero and the reconstruction bound holds.
    g = synth.misc_rng(18, 0)
    X = (g.uniform(1, 8, (2, 8, 8)) * np.sign(g.standard_normal((2, 8, 8)))
         * 2.0 ** -140).astype(np.float32)
    assert np.all(np.abs(X) < np.finfo(np.float32).tiny)
    Q, s, c = orc.quantize(X)
    assert np.all(s > 0) and np.all(c > 0)
    D = orc.dequantize(Q, s, c).astype(np.float64)
    assert np.all(np.abs(Q).max(axis=1) == 127)
    bound = s[:, :, None].astype(np.float64) * c[:, None, :] * (0.5 + 2.0 ** -10)
    # the dequantized product itself is subnormal: allow its quantum
    assert np.all(np.abs(D - X) <= bound + 2.0 ** -149)


def test_rounding_is_exhaustive_nearest_even(orc):
    # For every element, the code is the member of {-127..127} nearest to
    # the exact product t_ij = Y_ij * iota_j, ties to the even code, found by
    # trying all 255.  Y and iota are rebuilt from the stored scales with
    # numpy's IEEE fp32 ops; the product is taken exactly in fp64.
    X = _states(19, nh=3, dk=32, dv=32)
    Q, s, c = orc.quantize(X)
    s32 = s.astype(np.float32)
    with np.errstate(divide="ignore"):
        rho = np.where(s32 > 0, np.float32(1) / s32, np.float32(0)).astype(np.float32)
    Y = (X * rho[:, :, None]).astype(np.float32)
    m = np.abs(Y).max(axis=1)
    iota = np.where(m > 0, np.float32(127) / m, np.float32(0)).astype(np.float32)
    t = Y.astype(np.float64) * iota[:, None, :].astype(np.float64)
    codes = np.arange(-127, 128, dtype=np.float64)
    d = np.abs(t[..., None] - codes)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, codes, np.nan)
    # among equally near codes take the even one
    even = np.where(np.isnan(cand) | (np.mod(cand, 2) != 0), np.nan, cand)
    pick = np.where(np.isnan(even).all(-1), np.nanmax(cand, -1), np.nanmax(even, -1))
    assert np.array_equal(Q.astype(np.float64), pick)


def test_reciprocal_overflow_column_is_zero(orc):
    # A column whose largest smoothed magnitude is so small that 127/m
    # overflows fp32 is coded as a zero column.
    X = np.zeros((1, 2, 2), np.float32)
    X[0, 0, 0] = 1.0
    X[0, 0, 1] = np.float32(1e-44)
    X[0, 1, 0] = 1.0
    Q, s, c = orc.quantize(X)
    assert c[0, 1] == 0 and np.all(Q[0, :, 1] == 0)
    assert c[0, 0] > 0


# ------------------------------------------------------------- fp16 rows
def test_fp16_matches_ieee_conversion(orc):
    g = synth.misc_rng(20, 0)
    x = np.concatenate([
        g.standard_normal(20000) * 10.0 ** g.uniform(-9, 5, 20000),
        np.array([65504, 65505, 65519, 65520, 70000, 1e9, -65520, 6.1e-5, 6.09e-5, 5.96e-8,
                  2.98e-8, 2.99e-8, 1e-8, 0.0, -0.0, 1.0 + 2 ** -11, 1.0 + 3 * 2 ** -11]),
    ]).astype(np.float32)
    h = orc.f32_to_f16(x)
    ref = x.astype(np.float16)
    ref = np.where(np.isinf(ref), np.sign(ref) * np.float16(65504), ref).astype(np.float16)
    assert np.array_equal(h, ref.view(np.uint16))
    back = orc.f16_to_f32(h)
    assert np.array_equal(back, ref.astype(np.float32))


# ---------------------------------------------------------- DAMP layout
def _hp(seed, nh, dk, n_hp):
    g = synth.misc_rng(seed, 5)
    return np.stack([np.sort(g.choice(dk, n_hp, replace=False)) for _ in range(nh)]).astype(np.int32)


def test_damp_split_rows_and_codes(orc):
    nh, dk, dv, n_hp = 3, 16, 12, 3
    X = _states(21, nh, dk, dv)
    hp = _hp(21, nh, dk, n_hp)
    Qc, c, rows = orc.quantize_damp(X, hp)
    for h in range(nh):
        # hp rows are fp16 of X
        assert np.array_equal(rows[h], orc.f32_to_f16(X[h, hp[h]]))
        rest = np.setdiff1d(np.arange(dk), hp[h])
        # remaining rows: column-only INT8 over those rows only
        m = np.abs(X[h, rest]).max(axis=0)
        assert np.array_equal(np.abs(Qc[h]).max(axis=0), np.full(dv, 127))
        D = Qc[h].astype(np.float64) * c[h]
        assert np.all(np.abs(D - X[h, rest]) <= c[h] * (0.5 + 2 ** -10) + np.abs(X[h, rest]) * 2 ** -22)
        np.testing.assert_allclose(c[h], m / 127, rtol=2 ** -23)
    Xd = orc.dequantize_damp(Qc, c, rows, hp)
    for h in range(nh):
        assert np.array_equal(Xd[h, hp[h]], orc.f16_to_f32(rows[h]))


def test_damp_column_power_of_two_rescaling_absorbed(orc):
    # Figure 7 (LinQuant): per-channel scales absorb a consistent diagonal
    # rescaling.  Column-only codes are unchanged under 2^e_j column scaling.
    nh, dk, dv, n_hp = 2, 16, 12, 2
    X = _states(22, nh, dk, dv)
    hp = _hp(22, nh, dk, n_hp)
    e = synth.misc_rng(22, 1).integers(-5, 6, dv)
    Qa, ca, _ = orc.quantize_damp(X, hp)
    Qb, cb, _ = orc.quantize_damp(X * (2.0 ** e).astype(np.float32), hp)
    assert np.array_equal(Qa, Qb)
    assert np.array_equal(cb, ca * (2.0 ** e).astype(np.float32))
