"""GPU parity of the per-step decode paths through the C ABI:
fp32-state baseline (gdn_fp32_decode_step) and fused INT8 per-step decode
(gdn_quant_decode_step with W = 1, r = 0).

Bars (l2-relative per head):
  * o: 1e-4 with fp32 I/O; with bf16 output every element is a correct
    bf16 rounding of a value within fp32 error of the oracle, and per head
    the gap to the oracle's bf16-rounded output is <= 2e-3
    (tests/_gpu.check_outputs);
  * updated state before requantization: 1e-4;
  * fused requantization: codes and scales equal the oracle's codec
    applied to the kernel's own pre-quantization tensor, bit for bit;
  * codes against the oracle's own codes: differences are +-1 and only at
    elements whose pre-rounding value is within 1e-3 of a rounding tie.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu import (assert_encoding_is_oracle_codec, check_outputs, desc_for, dev, dev_io, host, host_io,
                        lib, near_tie_codes, per_head_rel, say, sub_cfg, torch_cuda)

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", dict()),                                   # 64x64, fp32 I/O, scalar gate
    ("prefix_cache", dict(B=2, H=5)),                   # 128x128 bf16, outliers
    ("prefix_cache", dict(B=1, H=6, decay="channel", a_lo=0.8)),
    ("prefix_cache", dict(B=1, H=6, dk=128, dv=64, io="f32")),
    ("prefix_cache", dict(B=1, H=6, dk=64, dv=128)),
]


def _state(cfg, nh, seed):
    if cfg.get("outlier_rows"):
        return synth.prefill_states(cfg, heads=range(nh))
    return synth.random_states(seed, nh, cfg["dk"], cfg["dv"])


def _ids(c):
    return f"{c[0]}-" + "-".join(f"{k}{v}" for k, v in c[1].items())


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_fp32_step(case):
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[case[0]], **case[1])
    nh = cfg["B"] * cfg["H"]
    bf = cfg["io"] == "bf16"
    d = desc_for(cfg, W=1, r=0)
    S = _state(cfg, nh, 11)
    inp = synth.step_inputs(cfg, 0)
    Sd = dev(S)
    o = torch.empty(nh * cfg["dv"], dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    say("fp32 step", case)
    g.gdn_fp32_decode_step(d, Sd, dev_io(inp, "q", bf), dev_io(inp, "k", bf), dev_io(inp, "v", bf),
                           dev(inp["a"]), dev(inp["b"]), o)
    torch.cuda.synchronize()
    S_ref, o_ref = oracle.recur(S, inp["q"][None], inp["k"][None], inp["v"][None], inp["a"][None],
                                inp["b"][None])
    check_outputs(host_io(o, bf), o_ref[0], bf)
    assert per_head_rel(host(Sd).reshape(S.shape), S_ref).max() <= 1e-5


@pytest.mark.parametrize("case", CASES, ids=_ids)
def test_fused_step_teacher_forced(case):
    """From the oracle's quantized state, one fused step on both sides."""
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[case[0]], **case[1])
    nh, dk, dv = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"]
    bf = cfg["io"] == "bf16"
    d = desc_for(cfg, W=1, r=0, flags=g.DEBUG_PREQUANT)
    S = _state(cfg, nh, 12)
    if not cfg.get("outlier_rows"):
        S *= np.float32(0.3)
    Q, s, c = oracle.quantize(S)
    st = g.alloc_state(d)
    st["codes"].copy_(torch.from_numpy(Q.reshape(-1)))
    st["row_scale"].copy_(torch.from_numpy(s.reshape(-1)))
    st["col_scale"].copy_(torch.from_numpy(c.reshape(-1)))
    inp = synth.step_inputs(cfg, 3)
    o = torch.empty(nh * dv, dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    say("fused step", case)
    g.gdn_quant_decode_step(d, st, dev_io(inp, "q", bf), dev_io(inp, "k", bf), dev_io(inp, "v", bf),
                            dev(inp["a"]), dev(inp["b"]), o, 0)
    torch.cuda.synchronize()
    ref = oracle.quant_step(Q, s, c, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    check_outputs(host_io(o, bf), ref["o"], bf)
    P = host(st["prequant_out"]).reshape(nh, dk, dv)
    assert per_head_rel(P, ref["S_pre"]).max() <= 1e-4
    # fused requantization == the oracle's codec on the kernel's own input
    assert_encoding_is_oracle_codec(P, host(st["codes"]), host(st["col_scale"]), host(st["row_scale"]))
    # and against the oracle's own codes: +-1 at near-ties only
    gQ = host(st["codes"]).reshape(nh, dk, dv).astype(np.int32)
    diff = gQ - ref["Q"].astype(np.int32)
    assert np.abs(diff).max() <= 1
    ties = near_tie_codes(ref["S_f32"], ref["s"], ref["c"], 1e-3)
    assert not np.any((diff != 0) & ~ties)
    np.testing.assert_allclose(host(st["row_scale"]).reshape(nh, dk), ref["s"], rtol=1e-5)
    np.testing.assert_allclose(host(st["col_scale"]).reshape(nh, dv), ref["c"], rtol=1e-5)


def test_tiny_trajectory():
    """Tiny workload end to end: 256 fused steps from S_0 = 0, fp32 I/O.

    Teacher-forced: before each step the GPU state is set to the oracle's
    quantized state and one step is compared.  Free-running: the GPU's own
    trajectory error against the unquantized fp64 trajectory must be within
    x[0.8, 1.25] of the oracle's own INT8 trajectory error (near-tie code
    flips make the two quantized trajectories part, by design)."""
    torch = torch_cuda()
    g = lib()
    cfg = synth.WORKLOADS["tiny"]
    nh, dk, dv, T = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["T"]
    d = desc_for(cfg)
    inp = synth.steps_inputs(cfg, 0, T)
    # oracle trajectories
    S_exact = np.zeros((nh, dk, dv))
    _, o_exact = oracle.recur(S_exact, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    Q = np.zeros((nh, dk, dv), np.int8)
    s = np.zeros((nh, dk), np.float32)
    c = np.zeros((nh, dv), np.float32)
    o_orc = np.empty((T, nh, dv))
    states = []
    for t in range(T):
        states.append((Q, s, c))
        r = oracle.quant_step(Q, s, c, inp["q"][t], inp["k"][t], inp["v"][t], inp["a"][t], inp["b"][t])
        Q, s, c, o_orc[t] = r["Q"], r["s"], r["c"], r["o"]
    # GPU free-running
    st = g.alloc_state(d)
    o = torch.empty(nh * dv, dtype=torch.float32, device="cuda")
    o_gpu = np.empty((T, nh, dv))
    say("tiny free-running")
    for t in range(T):
        g.gdn_quant_decode_step(d, st, dev(inp["q"][t]), dev(inp["k"][t]), dev(inp["v"][t]),
                                dev(inp["a"][t]), dev(inp["b"][t]), o, 0)
        o_gpu[t] = host(o).reshape(nh, dv)
    err_gpu = np.mean([per_head_rel(o_gpu[t], o_exact[t]).mean() for t in range(T)])
    err_orc = np.mean([per_head_rel(o_orc[t], o_exact[t]).mean() for t in range(T)])
    assert 0.8 <= err_gpu / err_orc <= 1.25, (err_gpu, err_orc)
    # teacher-forced every 16th step
    say("tiny teacher-forced")
    for t in range(0, T, 16):
        Qt, st_s, st_c = states[t]
        st["codes"].copy_(torch.from_numpy(Qt.reshape(-1)))
        st["row_scale"].copy_(torch.from_numpy(st_s.reshape(-1)))
        st["col_scale"].copy_(torch.from_numpy(st_c.reshape(-1)))
        g.gdn_quant_decode_step(d, st, dev(inp["q"][t]), dev(inp["k"][t]), dev(inp["v"][t]),
                                dev(inp["a"][t]), dev(inp["b"][t]), o, 0)
        assert per_head_rel(host(o).reshape(nh, dv), o_orc[t]).max() <= 1e-4
