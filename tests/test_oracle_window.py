"""Pins of the oracle's per-step quantized decode (c3), per-window decode
(c4), flush with Compensator Tokens (c5) and DAMP calibration (c6).

Sources: LeapQuant project page -- per-window quantization paragraph
(fixed low-bit state + buffered high-precision updates, full rebuild at the
window end), Compensator Tokens paragraph (high-precision outer products
removed before quantization, sharing the update path of real tokens),
residual-smoothing paragraph; DAMP abstract (error energy x decay
persistence picks the high-precision channels); LinQuant Table 3.
"""
import numpy as np
import pytest

import synth


def _steps(seed, n, nh, dk, dv, kda=False, a_lo=0.9):
    g = synth.misc_rng(seed, 11)
    q = g.standard_normal((n, nh, dk))
    k = g.standard_normal((n, nh, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((n, nh, dv))
    a = g.uniform(a_lo, 1.0, (n, nh, dk if kda else 1))
    b = g.uniform(0, 1, (n, nh))
    return [x.astype(np.float32) for x in (q, k, v, a, b)]


def _qstate(orc, seed, nh, dk, dv):
    X = synth.random_states(seed, nh, dk, dv)
    return orc.quantize(X)


@pytest.mark.parametrize("kda", [False, True])
def test_window_without_quantization_is_sequential(orc, kda):
    # With the fixed state exact, buffering updates and reading outputs from
    # fixed state + buffer is the sequential recurrence unrolled.
    nh, dk, dv, n = 3, 16, 12, 9
    q, k, v, a, b = _steps(1, n, nh, dk, dv, kda, 0.8)
    X0 = synth.random_states(1, nh, dk, dv).astype(np.float64)
    o_w, u_w, SW = orc.window(X0, q, k, v, a, b)
    S_seq, o_seq, u_seq = orc.recur(X0, q, k, v, a, b, want_u=True)
    np.testing.assert_allclose(o_w, o_seq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(u_w, u_seq, rtol=0, atol=1e-12)
    np.testing.assert_allclose(SW, S_seq, rtol=0, atol=1e-12)


@pytest.mark.parametrize("kda", [False, True])
def test_window_of_one_is_per_step_decode(orc, kda):
    nh, dk, dv = 4, 16, 16
    Q, s, c = _qstate(orc, 2, nh, dk, dv)
    q, k, v, a, b = _steps(2, 1, nh, dk, dv, kda)
    step = orc.quant_step(Q, s, c, q[0], k[0], v[0], a[0], b[0])
    X0 = orc.state_base(Q, s, c)
    o_w, _, SW = orc.window(X0, q, k, v, a, b)
    np.testing.assert_allclose(step["o"], o_w[0], rtol=0, atol=1e-12)
    np.testing.assert_allclose(step["S_pre"], SW, rtol=0, atol=1e-12)
    # the two separately written paths hand the same fp32 tensor to the
    # codec except where fp64 rounding order flips an fp32 rounding
    same = np.all(step["S_f32"] == SW.astype(np.float32), axis=(1, 2))
    Qw, sw, cw = orc.quantize(SW.astype(np.float32))
    for h in np.nonzero(same)[0]:
        assert np.array_equal(step["Q"][h], Qw[h]) and np.array_equal(step["s"][h], sw[h])
    assert same.sum() >= nh - 1


def test_zero_write_window_reads_decayed_fixed_state(orc):
    nh, dk, dv, n = 2, 16, 8, 6
    q, k, v, a, b = _steps(3, n, nh, dk, dv, True, 0.8)
    b[:] = 0.0
    X0 = synth.random_states(3, nh, dk, dv).astype(np.float64)
    o, u, SW = orc.window(X0, q, k, v, a, b)
    assert np.all(u == 0.0)
    G = np.cumprod(a.astype(np.float64), axis=0)            # [n, nh, dk]
    for t in range(n):
        np.testing.assert_allclose(o[t], np.einsum("hij,hi->hj", X0, G[t] * q[t]),
                                   rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(SW, G[-1][:, :, None] * X0, rtol=1e-14)


def test_identity_steps_requantize_to_a_fixed_point(orc):
    # a = 1, b = 0 is the identity: u = 0 exactly, the state only goes
    # through the codec again each step.  Every event stays within the
    # codec bound and the codes settle within a few steps.
    nh, dk, dv = 3, 16, 16
    Q, s, c = _qstate(orc, 4, nh, dk, dv)
    q, k, v, a, b = _steps(4, 1, nh, dk, dv)
    a[:] = 1.0
    b[:] = 0.0
    D0 = orc.dequantize(Q, s, c).astype(np.float64)
    hist = []
    for _ in range(8):
        prev = orc.dequantize(Q, s, c).astype(np.float64)
        out = orc.quant_step(Q, s, c, q[0], k[0], v[0], a[0], b[0])
        Q, s, c = out["Q"], out["s"], out["c"]
        D = orc.dequantize(Q, s, c).astype(np.float64)
        bound = s[:, :, None].astype(np.float64) * c[:, None, :] * (0.5 + 2 ** -10)
        assert np.all(np.abs(D - prev) <= bound + 2 ** -22 * np.abs(prev))
        hist.append(Q.copy())
    assert np.array_equal(hist[-1], hist[-2]) or np.array_equal(hist[-1], hist[-3])
    assert np.max(np.abs(D - D0)) < 0.05 * np.max(np.abs(D0))


# ------------------------------------------------------------------ flush
def _svd_top(R):
    U, S, Vt = np.linalg.svd(R)
    return S, U, Vt


def test_compensators_plus_residual_rebuild_state(orc):
    nh, dk, dv, r = 3, 16, 12, 3
    SW = synth.random_states(5, nh, dk, dv).astype(np.float64) * 3
    out = orc.compress(SW, r)
    C = np.einsum("hci,hcj->hij", out["p"].astype(np.float64), out["w"].astype(np.float64))
    # R is the fp64 residual rounded once to fp32
    resid = SW - C
    assert np.all(np.abs(out["R"] - resid) <= 2.0 ** -24 * np.abs(resid) + 1e-300)
    # the stored representation rebuilds S_W within the codec bound
    D = orc.dequantize(out["Q"], out["s"], out["c"]).astype(np.float64)
    bound = out["s"][:, :, None].astype(np.float64) * out["c"][:, None, :] * (0.5 + 2 ** -10)
    assert np.all(np.abs(SW - (C + D)) <= bound + 2.0 ** -22 * np.abs(resid) + 1e-12)
    # w vectors are unit
    np.testing.assert_allclose(np.linalg.norm(out["w"].astype(np.float64), axis=-1), 1.0, rtol=1e-6)


def test_compensators_match_svd_with_spectral_gap(orc):
    # With a clear gap, 20 power-iteration steps reach the leading singular
    # pairs: p_c w_c^T = sigma_c u_c v_c^T (LAPACK SVD, sign-free product).
    g = synth.misc_rng(6, 0)
    nh, dk, dv, r = 2, 16, 12, 2
    SW = np.empty((nh, dk, dv))
    for h in range(nh):
        U, _ = np.linalg.qr(g.standard_normal((dk, dk)))
        V, _ = np.linalg.qr(g.standard_normal((dv, dv)))
        sig = np.array([100.0, 10.0] + list(np.linspace(0.9, 0.1, dv - 2)))
        SW[h] = (U[:, :dv] * sig) @ V.T
    out = orc.compress(SW, r)
    for h in range(nh):
        S, U, Vt = _svd_top(SW[h])
        for ci in range(r):
            ref = S[ci] * np.outer(U[:, ci], Vt[ci])
            got = np.outer(out["p"][h, ci], out["w"][h, ci]).astype(np.float64)
            assert np.max(np.abs(got - ref)) <= 2e-6 * S[0]


def test_rank_one_state_leaves_tiny_residual(orc):
    g = synth.misc_rng(7, 0)
    nh, dk, dv = 2, 16, 12
    SW = np.einsum("hi,hj->hij", g.standard_normal((nh, dk)), g.standard_normal((nh, dv)))
    out = orc.compress(SW, 1)
    assert np.max(np.abs(out["R"])) <= 1e-6 * np.max(np.abs(SW))


def test_zero_state_gives_zero_compensators(orc):
    SW = np.zeros((2, 8, 8))
    out = orc.compress(SW, 2)
    assert np.all(out["p"] == 0) and np.all(out["w"] == 0)
    assert np.all(out["Q"] == 0) and np.all(out["s"] == 0) and np.all(out["c"] == 0)


def test_power_iteration_restarts_when_start_vector_is_annihilated(orc):
    # Rows of R sum to zero, so R 1 = 0 and the first iterate vanishes; the
    # iteration restarts from R's largest column and still finds the top
    # singular pair.
    g = synth.misc_rng(8, 0)
    dk, dv = 8, 6
    u = g.standard_normal(dk)
    v = g.standard_normal(dv)
    v -= v.mean()
    w = g.standard_normal(dv)
    w -= w.mean()
    w -= v * (w @ v) / (v @ v)
    SW = (10 * np.outer(u, v) + 0.5 * np.outer(g.standard_normal(dk), w))[None]
    out = orc.compress(SW, 1)
    S, U, Vt = _svd_top(SW[0])
    ref = S[0] * np.outer(U[:, 0], Vt[0])
    got = np.outer(out["p"][0, 0], out["w"][0, 0]).astype(np.float64)
    assert np.max(np.abs(got - ref)) <= 1e-5 * S[0]


# ------------------------------------------------------------ calibration
def _calib_inputs(seed, n, nh, dk, dv, kda):
    q, k, v, a, b = _steps(seed, n, nh, dk, dv, kda, 0.8)
    return k, v, a, b


def _energy(orc, S0, k, v, a, b):
    """Per-row quantization error energy and mean gate, rebuilt from the
    oracle's step and codec entry points."""
    n = k.shape[0]
    nh, dk, dv = S0.shape
    S = S0.astype(np.float64)
    E = np.zeros((nh, dk))
    for t in range(n):
        S, _ = orc.recur(S, None, k[t:t + 1], v[t:t + 1], a[t:t + 1], b[t:t + 1])
        X = S.astype(np.float32)
        empty = np.zeros((nh, 0), np.int32)
        Qc, c, rows = orc.quantize_damp(X, empty)
        D = orc.dequantize_damp(Qc, c, rows, empty).astype(np.float64)
        E += np.sum((S - D) ** 2, axis=2)
    abar = a.astype(np.float64).mean(axis=0)
    if abar.shape[-1] == 1:
        abar = np.repeat(abar, dk, axis=-1)
    return E, abar


@pytest.mark.parametrize("kda", [False, True])
def test_calibration_scores_and_brute_force_ranking(orc, kda):
    nh, dk, dv, n, n_hp = 3, 8, 8, 12, 3
    k, v, a, b = _calib_inputs(9, n, nh, dk, dv, kda)
    S0 = np.zeros((nh, dk, dv), np.float32)
    idx, score = orc.calibrate(S0, k, v, a, b, n_hp)
    E, abar = _energy(orc, S0, k, v, a, b)
    np.testing.assert_allclose(score, E / np.maximum(1 - abar, 1e-6), rtol=1e-12)
    for h in range(nh):
        # brute force over every n_hp-subset: the chosen set maximises the
        # summed score (ties would go to lower indices)
        import itertools
        best = max(itertools.combinations(range(dk), n_hp),
                   key=lambda cmb: (sum(score[h, list(cmb)]), [-i for i in cmb]))
        assert idx[h].tolist() == sorted(best)


def test_calibration_picks_planted_high_error_row(orc):
    nh, dk, dv, n, n_hp = 2, 16, 8, 16, 2
    k, v, a, b = _calib_inputs(10, n, nh, dk, dv, True)
    # make key channel 5 carry most of the state: large k component and a
    # gate close to one (long memory)
    k[:, :, 5] *= 8.0
    a[:, :, 5] = 0.999
    S0 = np.zeros((nh, dk, dv), np.float32)
    idx, _ = orc.calibrate(S0, k, v, a, b, n_hp)
    assert np.all(np.any(idx == 5, axis=1))


def test_scalar_decay_ranking_is_energy_ranking(orc):
    # With one gate per head the persistence factor is the same for every
    # row, so the score ranking is the error-energy ranking.
    nh, dk, dv, n = 2, 16, 8, 10
    k, v, a, b = _calib_inputs(11, n, nh, dk, dv, False)
    S0 = synth.random_states(11, nh, dk, dv)
    idx, score = orc.calibrate(S0, k, v, a, b, 4)
    E, _ = _energy(orc, S0, k, v, a, b)
    for h in range(nh):
        assert np.array_equal(np.argsort(-score[h], kind="stable"), np.argsort(-E[h], kind="stable"))


def test_power_iteration_restart_with_exact_pairs(orc):
    # Column pairs (c, -c) make every row sum to zero exactly, so the first
    # step vanishes for both compensators; the result still matches the SVD.
    g = synth.misc_rng(31, 1)
    dk, dv = 16, 12
    A = 10.0 * np.outer(g.standard_normal(dk), g.standard_normal(dv // 2))
    A += 0.1 * g.standard_normal((dk, dv // 2))
    X = np.zeros((1, dk, dv))
    X[0, :, 0::2] = A
    X[0, :, 1::2] = -A
    out = orc.compress(X, 2)
    S, U, Vt = _svd_top(X[0])
    for ci in range(2):
        ref = S[ci] * np.outer(U[:, ci], Vt[ci])
        got = np.outer(out["p"][0, ci], out["w"][0, ci]).astype(np.float64)
        assert np.max(np.abs(got - ref)) <= 1e-5 * S[0]
