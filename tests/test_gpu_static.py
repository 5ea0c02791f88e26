"""Static scales through the C ABI (calibrate_static_scales, and the
per-step decode / encode with GDNQ_STATIC_SCALES) against the oracle's
reading of the STEPQuant page (orc_fit_static, orc_quantize_static,
orc_quant_step_static).

Bars:
  * fit: row scales and their reciprocals within 2e-5 relative of the
    oracle's (the GPU's calibration trajectory is the fp32 recurrence, the
    oracle's the fp64 one rounded to fp32); each column's chosen range is the
    oracle's, or one whose weighted error in the oracle's own sums is within
    1e-3 relative of the oracle's least (a near-tie the two summation orders
    may break either way);
  * encode under fixed scales: codes equal the oracle's static codec on the
    same fp32 input, bit for bit (packed layouts included); scales untouched;
  * decode step under fixed scales (teacher-forced from the GPU's own codes):
    outputs with the per-step bars (tests/_gpu.check_outputs), the fp32
    tensor handed to the codec within 1e-4 of the oracle's, codes equal the
    oracle's static codec on that tensor bit for bit, and against the
    oracle's own codes +-1 only at near-ties; scales bit-for-bit unchanged.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu import (check_outputs, desc_for, dev, dev_io, host, host_io, lib, near_tie_codes, per_head_rel,
                        say, sub_cfg, torch_cuda)

pytestmark = pytest.mark.gpu


def _fit(cfg, bits, n, S0, seed_t=0):
    """GPU fit and oracle fit on the same calibration steps; returns
    (desc, state, gpu planes, oracle fit, inputs)."""
    torch = torch_cuda()
    g = lib()
    nh, dk, dv = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"]
    bf = cfg["io"] == "bf16"
    d = desc_for(cfg, W=1, r=0, bits=bits, flags=g.STATIC_SCALES)
    st = g.alloc_state(d)
    inp = synth.steps_inputs(cfg, seed_t, n)
    say("static fit", cfg["dk"], cfg["dv"], cfg["decay"], bits, n)
    g.calibrate_static_scales(d, dev(S0), dev_io(inp, "q", bf), dev_io(inp, "k", bf), dev_io(inp, "v", bf),
                              dev(inp["a"]), dev(inp["b"]), n, st)
    torch.cuda.synchronize()
    rs = host(st["row_scale"]).reshape(2, nh, dk)
    cs = host(st["col_scale"]).reshape(2, nh, dv)
    fit = oracle.fit_static(S0, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], bits=bits)
    return d, st, rs, cs, fit


def _check_fit(rs, cs, fit):
    np.testing.assert_allclose(rs[0], fit["s"], rtol=2e-5)
    np.testing.assert_allclose(rs[1], fit["rho"], rtol=2e-5)
    nh, dv = cs.shape[1:]
    # which candidate the GPU kept: the oracle candidate nearest to its scale
    rel = np.abs(fit["cand_c"] - cs[0][:, None, :]) / np.maximum(np.abs(fit["cand_c"]), 1e-30)
    kg = np.argmin(rel, axis=1)
    assert np.all(np.take_along_axis(rel, kg[:, None, :], axis=1) <= 2e-5)
    e = fit["err"]
    eg = np.take_along_axis(e, kg[:, None, :], axis=1)[:, 0]
    eo = np.take_along_axis(e, fit["choice"][:, None, :], axis=1)[:, 0]
    assert np.all(eg <= eo * (1 + 1e-3) + 1e-30), np.max(eg / np.maximum(eo, 1e-30))
    return float(np.mean(kg == fit["choice"]))


FIT_CASES = [(128, 128, "scalar", 8), (128, 128, "channel", 8), (64, 64, "scalar", 4), (128, 64, "scalar", 6)]


@pytest.mark.parametrize("dk,dv,decay,bits", FIT_CASES)
def test_static_fit(dk, dv, decay, bits):
    cfg = dict(B=1, H=4, dk=dk, dv=dv, io="bf16", decay=decay, a_lo=0.85, seed=61 + dk + bits, W=1, r=0)
    S0 = synth.random_states(13 + bits, 4, dk, dv, scale=0.3)
    _, _, rs, cs, fit = _fit(cfg, bits, 12, S0)
    same = _check_fit(rs, cs, fit)
    assert same >= 0.9, same


@pytest.mark.parametrize("bits", [8, 4])
def test_static_encode_bit_exact(bits):
    torch = torch_cuda()
    g = lib()
    cfg = dict(B=1, H=3, dk=128, dv=128, io="bf16", decay="scalar", a_lo=0.9, seed=71, W=1, r=0)
    S0 = synth.random_states(17, 3, 128, 128, scale=0.3)
    d, st, rs, cs, _ = _fit(cfg, bits, 8, S0)
    X = (S0 * 2).astype(np.float32)                             # elements beyond the fitted range
    before = (st["row_scale"].clone(), st["col_scale"].clone())
    say("static encode", bits)
    g.gdn_state_quantize(d, dev(X), st)
    torch.cuda.synchronize()
    Q = oracle.quantize_static(X, rs[1], cs[1], bits=bits)
    want = oracle.pack_codes(Q, bits) if bits != 8 else Q
    got = host(st["codes"]).reshape(want.shape).view(want.dtype)
    assert np.array_equal(got, want)
    assert torch.equal(before[0], st["row_scale"]) and torch.equal(before[1], st["col_scale"])
    assert np.abs(Q.astype(int)).max() == 2 ** (bits - 1) - 1   # saturation happens in this case


STEP_CASES = [("prefix_cache", dict(B=2, H=4), 8), ("prefix_cache", dict(B=1, H=4, decay="channel", a_lo=0.8), 8),
              ("tiny", dict(), 8), ("prefix_cache", dict(B=1, H=4), 4)]


@pytest.mark.parametrize("wl,over,bits", STEP_CASES)
def test_static_decode_steps(wl, over, bits):
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[wl], **over)
    nh, dk, dv = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"]
    bf = cfg["io"] == "bf16"
    S0 = synth.prefill_states(cfg, heads=range(nh)) if cfg.get("outlier_rows") else \
        synth.random_states(23, nh, dk, dv, scale=0.3)
    d, st, rs, cs, _ = _fit(cfg, bits, 8, S0, seed_t=100)
    d.flags |= g.DEBUG_PREQUANT
    st = g.alloc_state(d) | {k: st[k] for k in ("row_scale", "col_scale")}
    g.gdn_state_quantize(d, dev(S0), st)
    scales = (st["row_scale"].clone(), st["col_scale"].clone())
    s, rho, c, io = rs[0], rs[1], cs[0], cs[1]
    for t in range(3):
        codes = host(st["codes"])
        Qg = codes.reshape(nh, dk, dv) if bits == 8 else oracle.unpack_codes(codes.view(np.uint8).reshape(nh * dk, -1), dv,
                                                                             bits).reshape(nh, dk, dv)
        inp = synth.step_inputs(cfg, t)
        o = torch.empty(nh * dv, dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
        say("static step", wl, over, bits, t)
        g.gdn_quant_decode_step(d, st, dev_io(inp, "q", bf), dev_io(inp, "k", bf), dev_io(inp, "v", bf),
                                dev(inp["a"]), dev(inp["b"]), o, 0)
        torch.cuda.synchronize()
        ref = oracle.quant_step_static(Qg, s, c, rho, io, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], bits=bits)
        check_outputs(host_io(o, bf), ref["o"], bf)
        P = host(st["prequant_out"]).reshape(nh, dk, dv)
        assert per_head_rel(P, ref["S_f32"]).max() <= 1e-4
        own = oracle.quantize_static(P, rho, io, bits=bits)
        codes = host(st["codes"])
        got = codes.reshape(nh, dk, dv) if bits == 8 else oracle.unpack_codes(codes.view(np.uint8).reshape(nh * dk, -1), dv,
                                                                              bits).reshape(nh, dk, dv)
        assert np.array_equal(got, own)
        diff = got.astype(np.int32) - ref["Q"].astype(np.int32)
        assert np.abs(diff).max() <= 1
        assert not np.any((diff != 0) & ~near_tie_codes(ref["S_f32"], s, c, 1e-3))
        assert torch.equal(scales[0], st["row_scale"]) and torch.equal(scales[1], st["col_scale"])


def test_static_full_size_sampled():
    """prefix_cache (32768 states): fit over 4 calibration steps, encode,
    one static decode step; sampled heads against the oracle."""
    torch = torch_cuda()
    g = lib()
    cfg = synth.WORKLOADS["prefix_cache"]
    nh, dk, dv = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"]
    d = desc_for(cfg, W=1, r=0, flags=g.STATIC_SCALES)
    st = g.alloc_state(d)
    S0 = synth.prefill_states(cfg)
    cal = synth.steps_inputs(cfg, 200, 4)
    say("static full size fit")
    g.calibrate_static_scales(d, dev(S0), dev_io(cal, "q", True), dev_io(cal, "k", True), dev_io(cal, "v", True),
                              dev(cal["a"]), dev(cal["b"]), 4, st)
    g.gdn_state_quantize(d, dev(S0), st)
    torch.cuda.synchronize()
    Q0 = host(st["codes"]).reshape(nh, dk, dv)
    inp = synth.step_inputs(cfg, 0)
    o = torch.empty(nh * dv, dtype=torch.bfloat16, device="cuda")
    say("static full size step")
    g.gdn_quant_decode_step(d, st, dev_io(inp, "q", True), dev_io(inp, "k", True), dev_io(inp, "v", True),
                            dev(inp["a"]), dev(inp["b"]), o, 0)
    torch.cuda.synchronize()
    rs = host(st["row_scale"]).reshape(2, nh, dk)
    cs = host(st["col_scale"]).reshape(2, nh, dv)
    sel = np.array([0, 12345, nh - 1])
    fit = oracle.fit_static(S0[sel], cal["q"][:, sel], cal["k"][:, sel], cal["v"][:, sel], cal["a"][:, sel],
                            cal["b"][:, sel])
    _check_fit(rs[:, sel], cs[:, sel], fit)
    ref = oracle.quant_step_static(Q0[sel], rs[0][sel], cs[0][sel], rs[1][sel], cs[1][sel], inp["q"][sel],
                                   inp["k"][sel], inp["v"][sel], inp["a"][sel], inp["b"][sel])
    check_outputs(host_io(o, True).reshape(nh, dv)[sel], ref["o"], True)
    got = host(st["codes"]).reshape(nh, dk, dv)[sel].astype(np.int32)
    diff = got - ref["Q"].astype(np.int32)
    assert np.abs(diff).max() <= 1
    assert not np.any((diff != 0) & ~near_tie_codes(ref["S_f32"], rs[0][sel], cs[0][sel], 1e-3))
