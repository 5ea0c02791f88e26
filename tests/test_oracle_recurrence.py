"""Pins of the oracle's unquantized recurrence (c1) against facts the pages
and the mathematics fix, not against a retyped copy of its own loop.

Sources: LinQuant (Functional Invariances for Low-Precision Linear
Recurrences), appendix Table 3 (DeltaNet / Gated DeltaNet / KDA update
rules) and Table 1 (which invariances hold for which recurrence).
"""
from fractions import Fraction

import numpy as np
import pytest

import synth


def _inputs(seed, n, nh, dk, dv, kda=False, a_lo=0.9):
    g = synth.misc_rng(seed, 1)
    q = g.standard_normal((n, nh, dk))
    k = g.standard_normal((n, nh, dk))
    q /= np.linalg.norm(q, axis=-1, keepdims=True)
    k /= np.linalg.norm(k, axis=-1, keepdims=True)
    v = g.standard_normal((n, nh, dv))
    a = g.uniform(a_lo, 1.0, (n, nh, dk if kda else 1))
    b = g.uniform(0, 1, (n, nh))
    return [x.astype(np.float32) for x in (q, k, v, a, b)]


def test_delta_write_stores_v_exactly(orc):
    # With beta = 1 and a unit key the delta rule overwrites the value
    # stored under k: S_t^T k_t = v_t (Table 3, DeltaNet family).
    nh, dk, dv = 3, 16, 12
    q, k, v, a, b = _inputs(1, 1, nh, dk, dv)
    k64 = k.astype(np.float64)
    k = (k64 / np.linalg.norm(k64, axis=-1, keepdims=True)).astype(np.float32)
    b[:] = 1.0
    S0 = synth.random_states(1, nh, dk, dv)
    S, _ = orc.recur(S0, q, k, v, a, b)
    kk = k[0].astype(np.float64)
    norm2 = np.sum(kk * kk, axis=-1)          # fp32 k is unit only to ~1e-7
    back = np.einsum("hij,hi->hj", S, kk)
    # exact identity: S_t^T k = a S^T k (1 - |k|^2) + |k|^2 v
    prev = a[0].astype(np.float64)[:, :, None] * S0.astype(np.float64)
    expect = np.einsum("hij,hi->hj", prev, kk) * (1 - norm2)[:, None] + norm2[:, None] * v[0]
    np.testing.assert_allclose(back, expect, rtol=0, atol=1e-12)
    np.testing.assert_allclose(back, v[0], rtol=0, atol=1e-5)


def test_zero_write_only_decays(orc):
    nh, dk, dv = 2, 8, 8
    for kda in (False, True):
        q, k, v, a, b = _inputs(2, 1, nh, dk, dv, kda)
        b[:] = 0.0
        S0 = synth.random_states(2, nh, dk, dv)
        S, _ = orc.recur(S0, q, k, v, a, b)
        expect = a[0].astype(np.float64)[:, :, None] * S0.astype(np.float64)
        assert np.array_equal(S, expect)


def test_identity_step_leaves_state(orc):
    nh, dk, dv = 2, 8, 8
    q, k, v, a, b = _inputs(3, 4, nh, dk, dv)
    a[:] = 1.0
    b[:] = 0.0
    S0 = synth.random_states(3, nh, dk, dv)
    S, o = orc.recur(S0, q, k, v, a, b)
    assert np.array_equal(S, S0.astype(np.float64))
    np.testing.assert_allclose(o[-1], np.einsum("hij,hi->hj", S0.astype(np.float64), q[-1]), rtol=1e-12)


def test_kda_with_equal_gates_is_gdn(orc):
    nh, dk, dv, n = 3, 16, 8, 5
    q, k, v, a, b = _inputs(4, n, nh, dk, dv)
    a_vec = np.repeat(a, dk, axis=-1)
    S0 = synth.random_states(4, nh, dk, dv)
    S1, o1 = orc.recur(S0, q, k, v, a, b)
    S2, o2 = orc.recur(S0, q, k, v, a_vec, b)
    assert np.array_equal(S1, S2) and np.array_equal(o1, o2)


# ---- exact rational brute force, written in Table 3's own orientation -----
def _table3_step(St, q, k, v, alpha, beta, kda):
    """One step in LinQuant Table 3's form, state dv x dk, exact Fractions:
    GDN: S_t = alpha S (I - beta k k^T) + beta v k^T
    KDA: S_t = S diag(alpha) (I - beta k k^T) + beta v k^T
    returns (S_t, o_t = S_t q)."""
    dv, dk = len(St), len(St[0])
    if kda:
        Sd = [[St[j][i] * alpha[i] for i in range(dk)] for j in range(dv)]
    else:
        Sd = [[St[j][i] * alpha for i in range(dk)] for j in range(dv)]
    M = [[(1 if i == l else 0) - beta * k[i] * k[l] for l in range(dk)] for i in range(dk)]
    new = [[sum(Sd[j][i] * M[i][l] for i in range(dk)) + beta * v[j] * k[l] for l in range(dk)]
           for j in range(dv)]
    o = [sum(new[j][i] * q[i] for i in range(dk)) for j in range(dv)]
    return new, o


@pytest.mark.parametrize("kda", [False, True])
def test_fraction_brute_force_table3_form(orc, kda):
    dk = dv = 4
    n = 8
    q, k, v, a, b = _inputs(5, n, 1, dk, dv, kda)
    S0 = synth.random_states(5, 1, dk, dv)
    S, o = orc.recur(S0, q, k, v, a, b)
    F = lambda x: Fraction(float(x))
    St = [[F(S0[0, i, j]) for i in range(dk)] for j in range(dv)]   # transpose
    for t in range(n):
        alpha = [F(x) for x in a[t, 0]] if kda else F(a[t, 0, 0])
        St, ot = _table3_step(St, [F(x) for x in q[t, 0]], [F(x) for x in k[t, 0]],
                              [F(x) for x in v[t, 0]], alpha, F(b[t, 0]), kda)
        np.testing.assert_allclose(o[t, 0], [float(x) for x in ot], rtol=0, atol=1e-13)
    exact = np.array([[float(St[j][i]) for j in range(dv)] for i in range(dk)])
    np.testing.assert_allclose(S[0], exact, rtol=0, atol=1e-13)


def test_unit_gate_is_deltanet(orc):
    # Table 3: Gated DeltaNet with alpha = 1 is DeltaNet.
    dk = dv = 4
    n = 6
    q, k, v, a, b = _inputs(6, n, 1, dk, dv)
    a[:] = 1.0
    S0 = np.zeros((1, dk, dv), np.float32)
    S, o = orc.recur(S0, q, k, v, a, b)
    F = lambda x: Fraction(float(x))
    St = [[Fraction(0)] * dk for _ in range(dv)]
    for t in range(n):
        kk = [F(x) for x in k[t, 0]]
        beta = F(b[t, 0])
        M = [[(1 if i == l else 0) - beta * kk[i] * kk[l] for l in range(dk)] for i in range(dk)]
        St = [[sum(St[j][i] * M[i][l] for i in range(dk)) + beta * F(v[t, 0, j]) * kk[l]
               for l in range(dk)] for j in range(dv)]
    exact = np.array([[float(St[j][i]) for j in range(dv)] for i in range(dk)])
    np.testing.assert_allclose(S[0], exact, rtol=0, atol=1e-13)


# ---- Table 1 invariances (Gated DeltaNet column; KDA for the value side) ---
def _orth(g, d):
    m, _ = np.linalg.qr(g.standard_normal((d, d)))
    return m


def test_rotation_of_queries_and_keys_leaves_outputs(orc):
    # R_QK: the same rotation on q and k leaves the outputs of GDN unchanged
    # (state starts at zero so it rotates along).
    nh, dk, dv, n = 2, 8, 6, 6
    q, k, v, a, b = _inputs(7, n, nh, dk, dv)
    R = _orth(synth.misc_rng(7, 2), dk)
    q64, k64 = q.astype(np.float64), k.astype(np.float64)
    qr = (q64 @ R.T)
    kr = (k64 @ R.T)
    S0 = np.zeros((nh, dk, dv), np.float32)
    _, o1 = orc.recur(S0, q64, k64, v, a, b)
    # the oracle takes fp32 inputs: compare in exact arithmetic terms by
    # feeding both runs fp32-rounded vectors and allowing that rounding
    _, o2 = orc.recur(S0, qr, kr, v, a, b)
    np.testing.assert_allclose(o2, o1, rtol=0, atol=5e-6)


@pytest.mark.parametrize("kda", [False, True])
def test_value_rotation_and_scaling_commute(orc, kda):
    # R_V and D_V: rotating / rescaling v rotates / rescales every output.
    nh, dk, dv, n = 2, 8, 6, 6
    q, k, v, a, b = _inputs(8, n, nh, dk, dv, kda)
    g = synth.misc_rng(8, 3)
    Rv = _orth(g, dv)
    D = np.diag(2.0 ** g.integers(-3, 4, dv))           # exact in binary
    S0 = np.zeros((nh, dk, dv), np.float32)
    _, o = orc.recur(S0, q, k, v, a, b)
    _, oD = orc.recur(S0, q, k, (v.astype(np.float64) @ D.T).astype(np.float32), a, b)
    np.testing.assert_allclose(oD, o @ D.T, rtol=1e-13, atol=1e-14)
    vr = v.astype(np.float64) @ Rv.T
    _, oR = orc.recur(S0, q, k, vr.astype(np.float32), a, b)
    np.testing.assert_allclose(oR, o @ Rv.T, rtol=0, atol=5e-6)
