"""Pins of the oracle's static-scale codec and fit (STEPQuant page: key-row
and value-column scales fitted offline from the state distribution and each
key row's impact on the output error; the page gives no formula, the reading
is written at orc_fit_static).

What pins it, besides its own arithmetic:
  * candidate 0 (the full calibrated range) on a single calibration state is
    the dynamic codec of that state, bit for bit (scales and codes; 8, 6 and
    4 bits) -- the dynamic codec is pinned by test_oracle_codec.py;
  * codes saturate at +-Qb with the sign of X under a huge power-of-2 scale;
  * a power-of-4 rescaling moves between X and rho exactly;
  * the output weights decide the column range in a hand-built two-row case:
    with all weight on the large row the full range is kept (its element is
    exact only there), with all weight on the small row the chosen range is
    the one whose dequantized value of that row is nearest (checked through
    the codec and dequantizer, not the fit's error sums);
  * a step with a = 1, b = 0 under the scales of the current state keeps the
    codes and gives o = D(Q)^T q;
  * the chosen candidate's weighted error is never above candidate 0's;
  * a per-key-channel gate with all channels equal fits like the scalar gate.
"""
import numpy as np
import pytest

import oracle
import synth


def _identity_steps(S0, n, q=None, seed=0):
    """n steps with a = 1, b = 0 (the state stays S0); q random unless given."""
    nh, dk, dv = S0.shape
    g = synth.misc_rng(seed, 41)
    qs = g.standard_normal((n, nh, dk)).astype(np.float32) if q is None else np.broadcast_to(q, (n, nh, dk))
    k = g.standard_normal((n, nh, dk)).astype(np.float32)
    v = g.standard_normal((n, nh, dv)).astype(np.float32)
    a = np.ones((n, nh, 1), np.float32)
    b = np.zeros((n, nh), np.float32)
    return np.ascontiguousarray(qs, np.float32), k, v, a, b


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_full_range_candidate_is_the_dynamic_codec(bits):
    S0 = synth.random_states(3, 4, 16, 24, scale=2.0)
    S0[1, 3, :] = 0.0                       # a zero row
    S0[2, :, 5] = 0.0                       # a zero column
    fit = oracle.fit_static(S0, *_identity_steps(S0, 1), bits=bits)
    Q, s, c = oracle.quantize(S0, bits=bits)
    assert np.array_equal(fit["s"], s)
    assert np.array_equal(fit["cand_c"][:, 0], c)
    Qs = oracle.quantize_static(S0, fit["rho"], fit["cand_iota"][:, 0], bits=bits)
    assert np.array_equal(Qs, Q)


@pytest.mark.parametrize("bits", [8, 4])
def test_saturation_and_power_of_4(bits):
    S0 = synth.random_states(5, 2, 8, 8)
    fit = oracle.fit_static(S0, *_identity_steps(S0, 1), bits=bits)
    qb = 2 ** (bits - 1) - 1
    big = (S0 * np.float32(2.0 ** 40)).astype(np.float32)
    Qb = oracle.quantize_static(big, fit["rho"], fit["iota"], bits=bits)
    nz = S0 != 0
    assert np.array_equal(Qb[nz], (np.sign(S0[nz]) * qb).astype(np.int8))
    Q1 = oracle.quantize_static((S0 * 4).astype(np.float32), fit["rho"], fit["iota"], bits=bits)
    Q2 = oracle.quantize_static(S0, (fit["rho"] * 4).astype(np.float32), fit["iota"], bits=bits)
    assert np.array_equal(Q1, Q2)
    assert np.abs(Q1.astype(int)).max() <= qb


def test_output_weights_decide_the_range():
    S0 = np.array([[[1.0], [0.3]]], np.float32)              # dk = 2, dv = 1
    # all weight on row 0: only the full range makes its element exact
    fa = oracle.fit_static(S0, *_identity_steps(S0, 1, q=np.array([1.0, 0.0], np.float32)))
    assert fa["choice"][0, 0] == 0
    # all weight on row 1: the range whose dequantized row-1 value is nearest 0.3
    fb = oracle.fit_static(S0, *_identity_steps(S0, 1, q=np.array([0.0, 1.0], np.float32)))
    errs = []
    for k in range(9):
        Qk = oracle.quantize_static(S0, fb["rho"], fb["cand_iota"][:, k], bits=8)
        Xk = oracle.dequantize(Qk, fb["s"], fb["cand_c"][:, k])
        errs.append(abs(float(Xk[0, 1, 0]) - 0.3))
    assert fb["choice"][0, 0] == int(np.argmin(errs))
    assert fb["choice"][0, 0] != 0                          # the ranges differ for the two weightings


def test_identity_step_keeps_codes():
    S0 = synth.random_states(7, 3, 16, 16)
    Q, s, c = oracle.quantize(S0)
    fit = oracle.fit_static(oracle.dequantize(Q, s, c), *_identity_steps(S0, 1))
    g = synth.misc_rng(7, 3)
    q = g.standard_normal((3, 16)).astype(np.float32)
    k = g.standard_normal((3, 16)).astype(np.float32)
    v = g.standard_normal((3, 16)).astype(np.float32)
    r = oracle.quant_step_static(Q, s, c, fit["rho"], fit["cand_iota"][:, 0], q, k, v,
                                 np.ones((3, 1), np.float32), np.zeros(3, np.float32))
    assert np.array_equal(r["Q"], Q)
    D = oracle.dequantize(Q, s, c).astype(np.float64)
    assert np.allclose(r["o"], np.einsum("hij,hi->hj", D, q.astype(np.float64)), rtol=0, atol=1e-12)


def test_choice_never_worse_than_full_range():
    cfg = dict(B=1, H=3, dk=32, dv=32, io="f32", decay="scalar", a_lo=0.9, seed=9)
    inp = synth.steps_inputs(cfg, 0, 12)
    S0 = synth.random_states(9, 3, 32, 32)
    fit = oracle.fit_static(S0, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    e = fit["err"]
    chosen = np.take_along_axis(e, fit["choice"][:, None, :], axis=1)[:, 0]
    assert np.all(chosen <= e[:, 0])
    assert np.array_equal(fit["choice"], np.argmin(e, axis=1))
    assert np.array_equal(fit["c"], np.take_along_axis(fit["cand_c"], fit["choice"][:, None, :], axis=1)[:, 0])


def test_equal_channel_gates_fit_like_the_scalar_gate():
    cfg = dict(B=1, H=2, dk=16, dv=16, io="f32", decay="scalar", a_lo=0.8, seed=11)
    inp = synth.steps_inputs(cfg, 0, 6)
    S0 = synth.random_states(11, 2, 16, 16)
    f1 = oracle.fit_static(S0, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    a_ch = np.repeat(inp["a"], 16, axis=2)
    f2 = oracle.fit_static(S0, inp["q"], inp["k"], inp["v"], a_ch, inp["b"])
    for key in ("s", "rho", "c", "iota", "choice"):
        assert np.array_equal(f1[key], f2[key])
