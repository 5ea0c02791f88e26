"""GPU parity of the 6- and 4-bit states through the C ABI (desc.bits).

Same bars as the 8-bit paths, with the codes compared in their packed byte
layout:
  * codec: identical seeded fp32 input -> the packed codes equal the
    oracle's codes packed by the oracle, byte for byte; row and column
    scales bit-identical; the dequantized state bit-identical;
  * fused per-step decode, teacher-forced from the oracle's b-bit state:
    o by check_outputs, the pre-quantization state within 1e-4, the fused
    requantization equal to the oracle's codec on the kernel's own input
    byte for byte, and against the oracle's own codes +-1 only at near-ties;
  * window mode, teacher-forced from the oracle's b-bit window-start state:
    every o_t, the buffered u_t, the flush residual and compensators as for
    8 bits, the flush's codes equal to the oracle's codec on its residual.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu import (assert_encoding_is_oracle_codec, check_outputs, desc_for, dev, dev_io, host, host_io,
                        lib, near_tie_codes, per_head_rel, say, sub_cfg, torch_cuda)

pytestmark = pytest.mark.gpu

QMAX = {6: 31, 4: 7}


def _uneven(seed, nh, dk, dv):
    X = synth.random_states(seed, nh, dk, dv)
    g = synth.misc_rng(seed, 9)
    X *= (2.0 ** g.uniform(-8, 8, (nh, dk, 1))).astype(np.float32)
    X *= (2.0 ** g.uniform(-4, 4, (nh, 1, dv))).astype(np.float32)
    return X


def _ties(seed, nh, dk, dv, bits):
    # Every row holds 4 (row scale 2, reciprocal 1/2 exactly) and column
    # maxima Qb/8 (column reciprocal 16 exactly), so entries (2n+1)/16 land
    # on half-integers n + 1/2: round-half-even everywhere.
    qm = QMAX[bits]
    g = synth.misc_rng(seed, 3)
    X = (2.0 * g.integers(-qm, qm, (nh, dk, dv)) + 1.0) / 16.0
    X[:, :, 0] = 4.0
    X[:, 0, 1:] = qm / 8.0
    return X.astype(np.float32)


def _edge(seed, nh, dk, dv):
    X = _uneven(seed, nh, dk, dv)
    X[0] = 0
    X[1, 3, :] = 0
    X[1, :, 7] = 0
    X[2] *= np.float32(2.0 ** -140)
    X[3, 5, :] *= np.float32(1e30)
    X[4, :, 9] = np.float32(1e-44)
    X[5] = np.sign(X[5]) * np.float32(3.0e38)
    return X


def _packed(torch, Q, bits):
    return torch.from_numpy(oracle.pack_codes(Q, bits).view(np.int8).reshape(-1))


@pytest.mark.parametrize("bits", [6, 4])
@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("kind", ["uneven", "ties", "edge"])
def test_codec_bit_exact(bits, dk, dv, kind):
    torch = torch_cuda()
    g = lib()
    nh = 9
    X = {"uneven": lambda: _uneven(1, nh, dk, dv), "ties": lambda: _ties(2, nh, dk, dv, bits),
         "edge": lambda: _edge(3, nh, dk, dv)}[kind]()
    d = desc_for(dict(B=1, H=nh, dk=dk, dv=dv, W=1, r=0, decay="scalar", io="f32"), bits=bits)
    st = g.alloc_state(d)
    Xd = dev(X)
    say("lowbit codec", bits, dk, dv, kind)
    g.gdn_state_quantize(d, Xd, st)
    back = torch.empty_like(Xd)
    g.gdn_state_dequantize(d, st, back)
    torch.cuda.synchronize()
    Q, s, c = oracle.quantize(X, bits=bits)
    assert np.array_equal(host(st["codes"]).view(np.uint8), oracle.pack_codes(Q, bits).reshape(-1))
    assert np.array_equal(host(st["row_scale"]).reshape(nh, dk), s)
    assert np.array_equal(host(st["col_scale"]).reshape(nh, dv), c)
    ref = oracle.dequantize(Q, s, c)
    assert np.array_equal(host(back).reshape(nh, dk, dv).view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("bits", [6, 4])
@pytest.mark.parametrize("case", [
    ("prefix_cache", dict(B=2, H=5)),
    ("prefix_cache", dict(B=1, H=6, decay="channel", a_lo=0.8)),
    ("tiny", dict()),
], ids=["prefix", "prefix-kda", "tiny"])
def test_fused_step_teacher_forced(bits, case):
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[case[0]], **case[1])
    nh, dk, dv = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"]
    bf = cfg["io"] == "bf16"
    d = desc_for(cfg, W=1, r=0, flags=g.DEBUG_PREQUANT, bits=bits)
    S = (synth.prefill_states(cfg, heads=range(nh)) if cfg.get("outlier_rows")
         else synth.random_states(12, nh, dk, dv) * np.float32(0.3))
    Q, s, c = oracle.quantize(S, bits=bits)
    st = g.alloc_state(d)
    st["codes"].copy_(_packed(torch, Q, bits))
    st["row_scale"].copy_(torch.from_numpy(s.reshape(-1)))
    st["col_scale"].copy_(torch.from_numpy(c.reshape(-1)))
    inp = synth.step_inputs(cfg, 3)
    o = torch.empty(nh * dv, dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    say("lowbit fused step", bits, case)
    g.gdn_quant_decode_step(d, st, dev_io(inp, "q", bf), dev_io(inp, "k", bf), dev_io(inp, "v", bf),
                            dev(inp["a"]), dev(inp["b"]), o, 0)
    torch.cuda.synchronize()
    ref = oracle.quant_step(Q, s, c, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], bits=bits)
    check_outputs(host_io(o, bf), ref["o"], bf)
    P = host(st["prequant_out"]).reshape(nh, dk, dv)
    assert per_head_rel(P, ref["S_pre"]).max() <= 1e-4
    assert_encoding_is_oracle_codec(P, host(st["codes"]), host(st["col_scale"]), host(st["row_scale"]), bits=bits)
    gQ = oracle.unpack_codes(host(st["codes"]).view(np.uint8).reshape(nh, dk, -1), dv, bits).astype(np.int32)
    diff = gQ - ref["Q"].astype(np.int32)
    assert np.abs(diff).max() <= 1
    ties = near_tie_codes(ref["S_f32"], ref["s"], ref["c"], 1e-3)
    assert not np.any((diff != 0) & ~ties)


def _warm_state(cfg, nh, steps=48):
    inp = synth.steps_inputs(cfg, 0, steps, seed=cfg["seed"] + 100)
    S, _ = oracle.recur(np.zeros((nh, cfg["dk"], cfg["dv"])), inp["q"], inp["k"], inp["v"], inp["a"],
                        inp["b"])
    return S.astype(np.float32)


@pytest.mark.parametrize("bits", [6, 4])
@pytest.mark.parametrize("case", [
    ("gdn_serving", dict(B=1, H=6)),
    ("kda", dict(B=1, H=4)),
    ("gdn_serving", dict(B=1, H=4, dk=64, dv=64, io="f32")),
], ids=["serving", "kda", "serving-64-f32"])
def test_window_teacher_forced(bits, case):
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[case[0]], **case[1])
    nh, dk, dv, W, r = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"]
    bf = cfg["io"] == "bf16"
    d = desc_for(cfg, flags=g.DEBUG_PREQUANT, bits=bits)
    enc = oracle.compress(_warm_state(cfg, nh).astype(np.float64), r, 20, bits=bits)
    st = g.alloc_state(d)
    st["codes"].copy_(_packed(torch, enc["Q"], bits))
    st["row_scale"].copy_(torch.from_numpy(enc["s"].reshape(-1)))
    st["col_scale"].copy_(torch.from_numpy(enc["c"].reshape(-1)))
    st["comp_k"].copy_(torch.from_numpy(enc["p"].reshape(-1)))
    st["comp_v"].copy_(torch.from_numpy(enc["w"].reshape(-1)))
    inp = synth.steps_inputs(cfg, 0, W)
    odt = torch.bfloat16 if bf else torch.float32
    say("lowbit window", bits, case)
    outs = []
    for t in range(W):
        o = torch.empty(nh * dv, dtype=odt, device="cuda")
        one = {k: v[t] for k, v in inp.items()}
        g.gdn_quant_decode_step(d, st, dev_io(one, "q", bf), dev_io(one, "k", bf), dev_io(one, "v", bf),
                                dev(inp["a"][t]), dev(inp["b"][t]), o, t)
        outs.append(o)
    torch.cuda.synchronize()
    X0 = oracle.state_base(enc["Q"], enc["s"], enc["c"], enc["p"], enc["w"])
    o_ref, u_ref, SW = oracle.window(X0, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    for t in range(W):
        check_outputs(host_io(outs[t], bf), o_ref[t], bf)
    u_gpu = host(st["buf_u"]).reshape(nh, W, dv).transpose(1, 0, 2)
    assert per_head_rel(u_gpu.reshape(W * nh, dv), u_ref.reshape(W * nh, dv)).max() <= 1e-4
    say("lowbit flush", bits, case)
    g.gdn_quant_window_flush(d, st, W)
    torch.cuda.synchronize()
    ref = oracle.compress(SW, r, 20, bits=bits)
    scale = np.sqrt(np.sum(SW ** 2, axis=(1, 2)))
    R = host(st["prequant_out"]).reshape(nh, dk, dv).astype(np.float64)
    assert (np.sqrt(np.sum((R - ref["R"]) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
    p = host(st["comp_k"]).reshape(nh, r, dk).astype(np.float64)
    w = host(st["comp_v"]).reshape(nh, r, dv).astype(np.float64)
    C = np.einsum("hci,hcj->hij", p, w)
    Cr = np.einsum("hci,hcj->hij", ref["p"].astype(np.float64), ref["w"].astype(np.float64))
    assert (np.sqrt(np.sum((C - Cr) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
    assert_encoding_is_oracle_codec(R.astype(np.float32), host(st["codes"]), host(st["col_scale"]),
                                    host(st["row_scale"]), bits=bits)
