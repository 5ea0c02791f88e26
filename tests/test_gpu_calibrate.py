"""GPU parity of calibrate_scales (DAMP row selection) against the oracle.

Bars: row scores within 1e-3 relative (the GPU runs the recurrence in fp32,
the oracle in fp64; the error energy depends on codes that may round either
way at near-ties, which moves it by far less); the GPU's selection is
exactly the n_hp best of its own scores, ascending; it equals the oracle's
selection except where the two scores at the selection boundary are within
that tolerance (then both selections are correct)."""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu import desc_for, dev, dev_io, host, lib, say, sub_cfg, torch_cuda

pytestmark = pytest.mark.gpu


def _top(score, n):
    order = np.lexsort((np.arange(score.shape[-1]), -score))   # score desc, index asc
    return np.sort(order[:n])


@pytest.mark.parametrize("case", [
    ("damp", dict(B=1, H=6), 256),
    ("damp", dict(B=1, H=4, decay="scalar", a_lo=0.9), 64),
    ("damp", dict(B=1, H=4, dk=64, dv=64, io="f32", n_hp=4), 48),
], ids=["damp-kda", "damp-scalar", "damp-64-f32"])
def test_calibrate(case):
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[case[0]], **case[1])
    n = case[2]
    nh, dk, dv, n_hp = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["n_hp"]
    bf = cfg["io"] == "bf16"
    inp = synth.calib_inputs(cfg, n)
    S0 = np.zeros((nh, dk, dv), np.float32)
    d = desc_for(cfg)
    idx = torch.empty(nh * n_hp, dtype=torch.int32, device="cuda")
    score = torch.empty(nh * dk, dtype=torch.float32, device="cuda")
    say("calibrate", case)
    g.calibrate_scales(d, dev(S0), dev_io(inp, "k", bf), dev_io(inp, "v", bf), dev(inp["a"]), dev(inp["b"]),
                       n, idx, score)
    torch.cuda.synchronize()
    gi = host(idx).reshape(nh, n_hp)
    gs = host(score).reshape(nh, dk).astype(np.float64)
    ri, rs = oracle.calibrate(S0, inp["k"], inp["v"], inp["a"], inp["b"], n_hp)
    np.testing.assert_allclose(gs, rs, rtol=1e-3)
    for h in range(nh):
        assert gi[h].tolist() == _top(gs[h], n_hp).tolist()
        if gi[h].tolist() != ri[h].tolist():
            srt = np.sort(rs[h])[::-1]
            assert abs(srt[n_hp - 1] - srt[n_hp]) <= 2e-3 * srt[n_hp - 1], (h, gi[h], ri[h])


def test_calibrate_planted_row_and_nonzero_start():
    """A planted long-memory, large-key channel is always picked, also when
    calibration starts from a non-zero state."""
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS["damp"], B=1, H=3)
    nh, dk, dv, n_hp = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["n_hp"]
    n = 64
    inp = synth.calib_inputs(cfg, n)
    k = inp["k"].copy()
    a = inp["a"].copy()
    k[:, :, 17] *= 8.0
    a[:, :, 17] = 0.999
    k16 = synth.bf16_bits(k)
    k = synth.bf16_to_f32(k16)
    S0 = synth.random_states(9, nh, dk, dv, scale=0.1)
    d = desc_for(cfg)
    idx = torch.empty(nh * n_hp, dtype=torch.int32, device="cuda")
    say("calibrate planted")
    g.calibrate_scales(d, dev(S0), dev_io({"k16": k16}, "k", True), dev_io(inp, "v", True), dev(a),
                       dev(inp["b"]), n, idx, None)
    torch.cuda.synchronize()
    gi = host(idx).reshape(nh, n_hp)
    assert np.all(np.any(gi == 17, axis=1))
    ri, _ = oracle.calibrate(S0, k, inp["v"], a, inp["b"], n_hp)
    assert np.all(np.any(ri == 17, axis=1))
