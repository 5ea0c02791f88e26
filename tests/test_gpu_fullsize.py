"""Parity at the workloads' full sizes, in the launch configuration the
benchmark times (one workgroup per state, every state in one launch).  The
GPU runs every head; the oracle checks a sample of heads one by one (first,
last and seeded random ones), with the bars of the small-size tests."""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu import (assert_encoding_is_oracle_codec, check_outputs, desc_for, dev, dev_io, host, host_io,
                        lib, near_tie_codes, per_head_rel, say, torch_cuda)

pytestmark = pytest.mark.gpu


def _sample(nh, k=12, seed=0):
    g = synth.misc_rng(seed, 77)
    return np.unique(np.concatenate([[0, nh - 1], g.choice(nh, k, replace=False)]))


def _codes(st, nh, rows, dv, bits):
    """The GPU's packed codes of every head, unpacked by the oracle's layout."""
    P = host(st["codes"]).view(np.uint8).reshape(nh, rows, dv * bits // 8)
    return oracle.unpack_codes(P, dv, bits)


@pytest.mark.parametrize("bits", [8, 6, 4])
def test_prefix_cache_full_size(bits):
    """32768 pre-filled 128x128 states: quantize all, one fused per-step
    decode (b-bit codes) and one fp32-state step over all of them.  The
    step also writes its codec input (the same kernel: that store is a
    run-time branch), so the sampled heads' codes and scales are checked
    bit for bit against the oracle's codec on it."""
    torch = torch_cuda()
    g = lib()
    cfg = synth.WORKLOADS["prefix_cache"]
    nh, dk, dv = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"]
    heads = _sample(nh)
    S = synth.prefill_states(cfg)
    d = desc_for(cfg, bits=bits, flags=g.DEBUG_PREQUANT)
    st = g.alloc_state(d)
    Sd = dev(S)
    say("prefix_cache full: quantize", bits)
    g.gdn_state_quantize(d, Sd, st)
    torch.cuda.synchronize()
    Q, s, c = oracle.quantize(S[heads], bits=bits)
    assert np.array_equal(_codes(st, nh, dk, dv, bits)[heads], Q)
    assert np.array_equal(host(st["row_scale"]).reshape(nh, dk)[heads], s)
    assert np.array_equal(host(st["col_scale"]).reshape(nh, dv)[heads], c)
    inp = synth.step_inputs(cfg, 0)
    args = [dev_io(inp, "q", True), dev_io(inp, "k", True), dev_io(inp, "v", True), dev(inp["a"]),
            dev(inp["b"])]
    o = torch.empty(nh * dv, dtype=torch.bfloat16, device="cuda")
    say("prefix_cache full: fused step", bits)
    g.gdn_quant_decode_step(d, st, *args, o, 0)
    torch.cuda.synchronize()
    sub = {k: v[heads] for k, v in inp.items()}
    ref = oracle.quant_step(Q, s, c, sub["q"], sub["k"], sub["v"], sub["a"], sub["b"], bits=bits)
    check_outputs(host_io(o, True).reshape(nh, dv)[heads], ref["o"], True)
    hidx = torch.from_numpy(heads).cuda()
    P = host(st["prequant_out"].view(nh, dk * dv)[hidx]).reshape(len(heads), dk, dv)
    assert per_head_rel(P, ref["S_pre"]).max() <= 1e-4
    assert_encoding_is_oracle_codec(P, host(st["codes"].view(nh, -1)[hidx]), host(st["col_scale"].view(nh, dv)[hidx]),
                                    host(st["row_scale"].view(nh, dk)[hidx]), bits=bits)
    gQ = _codes(st, nh, dk, dv, bits)[heads].astype(np.int32)
    diff = gQ - ref["Q"].astype(np.int32)
    assert np.abs(diff).max() <= 1
    assert not np.any((diff != 0) & ~near_tie_codes(ref["S_f32"], ref["s"], ref["c"], 1e-3))
    np.testing.assert_allclose(host(st["row_scale"]).reshape(nh, dk)[heads], ref["s"], rtol=1e-5)
    if bits != 8:
        return
    # fp32-state baseline over all heads
    of = torch.empty(nh * dv, dtype=torch.bfloat16, device="cuda")
    say("prefix_cache full: fp32 step")
    g.gdn_fp32_decode_step(d, Sd, *args, of)
    torch.cuda.synchronize()
    S_ref, o_ref = oracle.recur(S[heads], sub["q"][None], sub["k"][None], sub["v"][None], sub["a"][None],
                                sub["b"][None])
    check_outputs(host_io(of, True).reshape(nh, dv)[heads], o_ref[0], True)
    assert per_head_rel(host(Sd).reshape(nh, dk, dv)[heads], S_ref).max() <= 1e-5


@pytest.mark.parametrize("name,bits", [("gdn_serving", 8), ("kda", 8), ("damp", 8), ("gdn_serving", 6),
                                       ("kda", 4)])
def test_window_full_size(name, bits):
    """All B*H heads of the window workloads: one full window and its flush.
    Every head starts from a seeded random state encoded by the GPU; the
    sampled heads are overwritten with the oracle's encoding of the same
    state so both sides start identical there."""
    torch = torch_cuda()
    g = lib()
    cfg = synth.WORKLOADS[name]
    nh, dk, dv, W, r = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"]
    n_hp = cfg.get("n_hp", 0)
    heads = _sample(nh, 8)
    S = synth.random_states(cfg["seed"], nh, dk, dv, scale=0.3)
    hp = None
    d = desc_for(cfg, flags=g.DEBUG_PREQUANT, bits=bits)
    st = g.alloc_state(d)
    if n_hp:
        gr = synth.misc_rng(cfg["seed"], 5)
        hp = np.stack([np.sort(gr.choice(dk, n_hp, replace=False)) for _ in range(nh)]).astype(np.int32)
        st["hp_idx"].copy_(torch.from_numpy(hp.reshape(-1)))
    say(name, "full: quantize", bits)
    g.gdn_state_quantize(d, dev(S), st)
    enc = oracle.compress(S[heads].astype(np.float64), r, 20, hp_idx=None if hp is None else hp[heads],
                          bits=bits)
    rows = dk - n_hp
    codes = st["codes"].view(nh, rows * dv * bits // 8)
    codes[torch.from_numpy(heads).cuda()] = torch.from_numpy(
        oracle.pack_codes(enc["Q"], bits).view(np.int8).reshape(len(heads), -1)).cuda()
    hidx = torch.from_numpy(heads).cuda()
    st["col_scale"].view(nh, dv)[hidx] = torch.from_numpy(enc["c"]).cuda()
    if hp is None:
        st["row_scale"].view(nh, dk)[hidx] = torch.from_numpy(enc["s"]).cuda()
    else:
        st["hp_rows"].view(nh, n_hp * dv)[hidx] = torch.from_numpy(
            enc["hp_rows"].view(np.int16).reshape(len(heads), -1)).cuda()
    st["comp_k"].view(nh, r * dk)[hidx] = torch.from_numpy(enc["p"].reshape(len(heads), -1)).cuda()
    st["comp_v"].view(nh, r * dv)[hidx] = torch.from_numpy(enc["w"].reshape(len(heads), -1)).cuda()
    inp = synth.steps_inputs(cfg, 0, W)
    outs = []
    say(name, "full: window", bits)
    for t in range(W):
        one = {k: v[t] for k, v in inp.items()}
        o = torch.empty(nh * dv, dtype=torch.bfloat16, device="cuda")
        g.gdn_quant_decode_step(d, st, dev_io(one, "q", True), dev_io(one, "k", True), dev_io(one, "v", True),
                                dev(one["a"]), dev(one["b"]), o, t)
        outs.append(o)
    g.gdn_quant_window_flush(d, st, W)
    torch.cuda.synchronize()
    sub = {k: v[:, heads] for k, v in inp.items()}
    if hp is None:
        X0 = oracle.state_base(enc["Q"], enc["s"], enc["c"], enc["p"], enc["w"])
    else:
        X0 = oracle.state_base(enc["Q"], None, enc["c"], enc["p"], enc["w"], hp_idx=hp[heads],
                               hp_rows=enc["hp_rows"])
    o_ref, _, SW = oracle.window(X0, sub["q"], sub["k"], sub["v"], sub["a"], sub["b"])
    for t in range(W):
        check_outputs(host_io(outs[t], True).reshape(nh, dv)[heads], o_ref[t], True)
    ref = oracle.compress(SW, r, 20, hp_idx=None if hp is None else hp[heads], bits=bits)
    scale = np.sqrt(np.sum(SW ** 2, axis=(1, 2)))
    hidx = torch.from_numpy(heads).cuda()
    R = host(st["prequant_out"].view(nh, dk * dv)[hidx]).reshape(len(heads), dk, dv)
    assert (np.sqrt(np.sum((R.astype(np.float64) - ref["R"]) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
    # the flush's codes on the sampled heads: the oracle's codec on its residual
    assert_encoding_is_oracle_codec(R, host(st["codes"].view(nh, -1)[hidx]), host(st["col_scale"].view(nh, dv)[hidx]),
                                    None if hp is not None else host(st["row_scale"].view(nh, dk)[hidx]), bits=bits,
                                    hp_idx=None if hp is None else hp[heads],
                                    hp_rows=None if hp is None else host(st["hp_rows"].view(nh, -1)[hidx]))
