"""Pins of the oracle's 6- and 4-bit states: the layout-0 codec with code
width b (codes in [-Qb, Qb], Qb = 2^(b-1) - 1; column scale m/Qb) and the
packed byte layouts (4 bits: two's complement nibbles, even column low; 6
bits: a 48-bit record per block of 8 columns, its low 32 bits in a first
plane, its high 16 bits in a second).

Source: LeapQuant project page, accuracy table (LeapQuant at 8, 6 and 4
bits).  The code range, the scale and the packing are readings: the pages
give no format.  The pins are hand-worked examples, byte layouts written by
hand, an exhaustive nearest-code search, closed-form relations to the 8-bit
codec, and invariants of the decode that do not depend on the code width.
"""
import numpy as np
import pytest

import synth

QMAX = {8: 127, 6: 31, 4: 7}


def _states(seed, nh=4, dk=16, dv=24):
    X = synth.random_states(seed, nh, dk, dv, 1.0)
    g = synth.misc_rng(seed, 9)
    X *= (2.0 ** g.uniform(-6, 6, (nh, dk, 1))).astype(np.float32)
    X *= (2.0 ** g.uniform(-3, 3, (nh, 1, dv))).astype(np.float32)
    return X


def test_hand_worked_4bit(orc):
    # Rows [4, y]: s = 2, rho = 1/2 exactly, Y = [2, y/2].  Column 0: m = 2,
    # iota = 7/2 exactly, every t = 7.  Column 1: m = 7/4, iota = 4 and
    # c = 1/4 exactly; t = 2y: 7, 2.5 (tie -> 2), 3.5 (tie -> 4), -2.5 (-> -2).
    X = np.array([[[4.0, 3.5], [4.0, 1.25], [4.0, 1.75], [4.0, -1.25]]], np.float32)
    Q, s, c = orc.quantize(X, bits=4)
    assert Q[0].tolist() == [[7, 7], [7, 2], [7, 4], [7, -2]]
    assert c[0, 1] == np.float32(0.25)
    assert c[0, 0] == np.float32(np.float32(2.0) / np.float32(7.0))


def test_hand_worked_6bit(orc):
    # Column 1: m = 31/16, iota = 16 and c = 1/16 exactly; t = 8y:
    # 31, 2.5 (tie -> 2), 3.5 (tie -> 4), -2.5 (-> -2).
    X = np.array([[[4.0, 31 / 8], [4.0, 5 / 16], [4.0, 7 / 16], [4.0, -5 / 16]]], np.float32)
    Q, s, c = orc.quantize(X, bits=6)
    assert Q[0].tolist() == [[31, 31], [31, 2], [31, 4], [31, -2]]
    assert c[0, 1] == np.float32(1 / 16)


@pytest.mark.parametrize("bits", [6, 4])
def test_code_range_full_scale_and_shared_row_scales(orc, bits):
    X = _states(31)
    Q, s, c = orc.quantize(X, bits=bits)
    Q8, s8, c8 = orc.quantize(X, bits=8)
    qm = QMAX[bits]
    assert Q.min() >= -qm and Q.max() <= qm
    assert np.all(np.abs(Q).max(axis=1) == qm)
    # the smoothing does not depend on the code width; the column scales
    # are the same column maxima over a different number of levels
    assert np.array_equal(s, s8)
    np.testing.assert_allclose(c.astype(np.float64) * qm, c8.astype(np.float64) * 127, rtol=2.0 ** -22)


@pytest.mark.parametrize("bits", [6, 4])
def test_reconstruction_bound(orc, bits):
    X = _states(32, nh=6)
    Q, s, c = orc.quantize(X, bits=bits)
    D = orc.dequantize(Q, s, c).astype(np.float64)
    err = np.abs(D - X)
    bound = s[:, :, None].astype(np.float64) * c[:, None, :] * (0.5 + 2.0 ** -10)
    assert np.all(err <= bound + np.abs(X) * 2.0 ** -22)
    assert np.max(err / bound) > 0.45


@pytest.mark.parametrize("bits", [6, 4])
def test_rounding_is_exhaustive_nearest_even(orc, bits):
    X = _states(33, nh=3, dk=32, dv=32)
    Q, s, c = orc.quantize(X, bits=bits)
    qm = QMAX[bits]
    with np.errstate(divide="ignore"):
        rho = np.where(s > 0, np.float32(1) / s, np.float32(0)).astype(np.float32)
    Y = (X * rho[:, :, None]).astype(np.float32)
    m = np.abs(Y).max(axis=1)
    iota = np.where(m > 0, np.float32(qm) / m, np.float32(0)).astype(np.float32)
    t = Y.astype(np.float64) * iota[:, None, :].astype(np.float64)
    codes = np.arange(-qm, qm + 1, dtype=np.float64)
    d = np.abs(t[..., None] - codes)
    best = d.min(axis=-1, keepdims=True)
    cand = np.where(d == best, codes, np.nan)
    even = np.where(np.isnan(cand) | (np.mod(cand, 2) != 0), np.nan, cand)
    pick = np.where(np.isnan(even).all(-1), np.nanmax(cand, -1), np.nanmax(even, -1))
    assert np.array_equal(Q.astype(np.float64), pick)


def test_pack_bytes_written_by_hand(orc):
    q4 = np.array([[1, -1, 7, -7, 0, 3, -4, 2]], np.int8)
    assert orc.pack_codes(q4, 4).tolist() == [[0xF1, 0x97, 0x30, 0x2C]]
    q6 = np.array([[1, -1, 31, -31, 16, -16, 0, 5]], np.int8)
    # 6-bit fields 01 3F 1F 21 10 30 00 05 at record bits 0, 6, ..., 42:
    # record 0x140C_1085FFC1 -> plane 1: C1 FF 85 10, plane 2: 0C 14
    assert orc.pack_codes(q6, 6).tolist() == [[0xC1, 0xFF, 0x85, 0x10, 0x0C, 0x14]]
    assert orc.pack_codes(q4, 8).view(np.int8).tolist() == q4.tolist()


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_pack_round_trip_every_code(orc, bits):
    qm = QMAX[bits]
    g = synth.misc_rng(34, bits)
    Q = g.integers(-qm, qm + 1, (5, 7, 128)).astype(np.int8)
    Q.reshape(-1)[: 2 * qm + 1] = np.arange(-qm, qm + 1)  # every code at least once
    Q[1, 2, 37] = 0
    P = orc.pack_codes(Q, bits)
    assert P.shape == (5, 7, 128 * bits // 8)
    assert np.array_equal(orc.unpack_codes(P, 128, bits), Q)
    # each column's code lives in its own bits: changing one code changes
    # only the bytes that hold it
    Q2 = Q.copy()
    Q2[1, 2, 37] = -1       # 0 -> -1 flips every bit of its field, in both planes
    diff = np.argwhere(orc.pack_codes(Q2, bits) != P)
    # column 37 = block 4, field 5: record bits 30..35 (plane 1 byte 19, plane 2 byte 64 + 8)
    expect = {8: [37], 4: [18], 6: [19, 64 + 8]}[bits]
    assert sorted(diff[:, 2].tolist()) == expect and np.all(diff[:, :2] == [1, 2])


@pytest.mark.parametrize("bits", [6, 4])
def test_decode_step_output_does_not_depend_on_code_width(orc, bits):
    # The per-step decode reads the given (Q, s, c) and takes o and the
    # updated state before requantizing: from the same stored state both
    # widths give the same o and the same fp32 tensor to the codec, whose
    # b-bit codes then equal the stand-alone codec's.
    cfg = dict(synth.WORKLOADS["tiny"], H=3)
    nh, dk, dv = 3, cfg["dk"], cfg["dv"]
    X = _states(35, nh=nh, dk=dk, dv=dv)
    Q, s, c = orc.quantize(X, bits=bits)
    inp = synth.step_inputs(cfg, 0)
    r8 = orc.quant_step(Q, s, c, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], bits=8)
    rb = orc.quant_step(Q, s, c, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], bits=bits)
    assert np.array_equal(r8["o"], rb["o"]) and np.array_equal(r8["S_f32"], rb["S_f32"])
    Qb, sb, cb = orc.quantize(rb["S_f32"], bits=bits)
    assert np.array_equal(rb["Q"], Qb) and np.array_equal(rb["s"], sb) and np.array_equal(rb["c"], cb)
    assert np.abs(rb["Q"]).max() <= QMAX[bits]


@pytest.mark.parametrize("bits", [6, 4])
def test_compress_compensators_do_not_depend_on_code_width(orc, bits):
    SW = _states(36, nh=3, dk=32, dv=32).astype(np.float64)
    e8 = orc.compress(SW, 2, 20, bits=8)
    eb = orc.compress(SW, 2, 20, bits=bits)
    assert np.array_equal(e8["p"], eb["p"]) and np.array_equal(e8["w"], eb["w"])
    assert np.array_equal(e8["R"], eb["R"])
    Qb, sb, cb = orc.quantize(eb["R"], bits=bits)
    assert np.array_equal(eb["Q"], Qb) and np.array_equal(eb["c"], cb)
