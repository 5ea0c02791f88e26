"""GPU parity of per-window decode (gdn_quant_decode_step in window mode)
and the window flush (gdn_quant_window_flush), through the C ABI.

Teacher-forced per window: both sides start from the same quantized
window-start state (the oracle's encoding of a warmed-up state, uploaded
to the GPU), run the same n tokens and flush.  Bars:
  * every o_t: check_outputs (1e-4 fp32 I/O; bf16 rounding bound);
  * buffered u_t: l2-relative 1e-4;
  * the residual handed to the codec (fp32, after the new compensators)
    and the compensator products: within 1e-4 of |S_W| per head (S_W, the
    rebuilt pre-compensator state, is the scale because S_W - p w^T
    cancels);
  * codes / scales / fp16 rows equal the oracle codec's output on that
    residual bit for bit.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu import (assert_encoding_is_oracle_codec, check_outputs, desc_for, dev, dev_io, host, host_io,
                        lib, per_head_rel, say, sub_cfg, torch_cuda)

pytestmark = pytest.mark.gpu


def _warm_state(cfg, nh, steps=48, seed_shift=100):
    """A state reached by the fp64 recurrence from zero (oracle), fp32."""
    inp = synth.steps_inputs(cfg, 0, steps, seed=cfg["seed"] + seed_shift)
    S, _ = oracle.recur(np.zeros((nh, cfg["dk"], cfg["dv"])), inp["q"], inp["k"], inp["v"], inp["a"],
                        inp["b"])
    return S.astype(np.float32)


def _hp_rows(cfg, nh, seed=7):
    g = synth.misc_rng(seed, 1)
    return np.stack([np.sort(g.choice(cfg["dk"], cfg["n_hp"], replace=False))
                     for _ in range(nh)]).astype(np.int32)


def _upload(torch, st, enc, hp):
    st["codes"].copy_(torch.from_numpy(np.ascontiguousarray(enc["Q"]).reshape(-1)))
    if st["row_scale"] is not None:
        st["row_scale"].copy_(torch.from_numpy(enc["s"].reshape(-1)))
    st["col_scale"].copy_(torch.from_numpy(enc["c"].reshape(-1)))
    if st["comp_k"] is not None:
        st["comp_k"].copy_(torch.from_numpy(enc["p"].reshape(-1)))
        st["comp_v"].copy_(torch.from_numpy(enc["w"].reshape(-1)))
    if hp is not None:
        st["hp_idx"].copy_(torch.from_numpy(hp.reshape(-1)))
        st["hp_rows"].copy_(torch.from_numpy(enc["hp_rows"].view(np.int16).reshape(-1)))


def _base(enc, hp):
    if hp is None:
        return oracle.state_base(enc["Q"], enc["s"], enc["c"], enc["p"], enc["w"])
    return oracle.state_base(enc["Q"], None, enc["c"], enc["p"], enc["w"], hp_idx=hp, hp_rows=enc["hp_rows"])


def _assert_oracle_encoding(st, R, hp):
    assert_encoding_is_oracle_codec(R.astype(np.float32), host(st["codes"]), host(st["col_scale"]),
                                    None if hp is not None else host(st["row_scale"]), hp_idx=hp,
                                    hp_rows=None if hp is None else host(st["hp_rows"]))


def _run_gpu_window(torch, g, d, st, inp, n, bf, o_dtype):
    nh = d.nh
    outs = []
    for t in range(n):
        o = torch.empty(nh * d.dv, dtype=o_dtype, device="cuda")
        g.gdn_quant_decode_step(d, st, dev_io({k: v[t] for k, v in inp.items()}, "q", bf),
                                dev_io({k: v[t] for k, v in inp.items()}, "k", bf),
                                dev_io({k: v[t] for k, v in inp.items()}, "v", bf),
                                dev(inp["a"][t]), dev(inp["b"][t]), o, t)
        outs.append(o)
    return outs


WCASES = [
    ("gdn_serving", dict(B=1, H=6), None),
    ("gdn_serving", dict(B=1, H=6), 5),                          # partial window
    ("kda", dict(B=1, H=4), None),
    ("damp", dict(B=1, H=4), None),
    ("gdn_serving", dict(B=1, H=4, dk=64, dv=64, io="f32", W=8, r=1), None),
    ("kda", dict(B=1, H=4, dk=128, dv=64, io="f32", W=6, r=3), None),
    ("damp", dict(B=1, H=4, dk=64, dv=128, W=4, r=2, n_hp=4), None),
]


def _wid(c):
    return f"{c[0]}-" + "-".join(f"{k}{v}" for k, v in c[1].items()) + f"-n{c[2]}"


@pytest.mark.parametrize("case", WCASES, ids=_wid)
def test_window_teacher_forced(case):
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[case[0]], **case[1])
    nh, dk, dv, W, r = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"]
    n = case[2] or W
    bf = cfg["io"] == "bf16"
    hp = _hp_rows(cfg, nh) if cfg.get("n_hp") else None
    d = desc_for(cfg, flags=g.DEBUG_PREQUANT)
    enc = oracle.compress(_warm_state(cfg, nh).astype(np.float64), r, 20, hp_idx=hp)
    st = g.alloc_state(d)
    _upload(torch, st, enc, hp)
    inp = synth.steps_inputs(cfg, 0, n)
    say("window", case)
    outs = _run_gpu_window(torch, g, d, st, inp, n, bf, torch.bfloat16 if bf else torch.float32)
    torch.cuda.synchronize()
    X0 = _base(enc, hp)
    o_ref, u_ref, SW = oracle.window(X0, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    for t in range(n):
        check_outputs(host_io(outs[t], bf), o_ref[t], bf)
    u_gpu = host(st["buf_u"]).reshape(nh, W, dv)[:, :n].transpose(1, 0, 2)
    assert per_head_rel(u_gpu.reshape(n * nh, dv), u_ref.reshape(n * nh, dv)).max() <= 1e-4
    say("flush", case)
    g.gdn_quant_window_flush(d, st, n)
    torch.cuda.synchronize()
    ref = oracle.compress(SW, r, 20, hp_idx=hp)
    scale = np.sqrt(np.sum(SW ** 2, axis=(1, 2)))
    R = host(st["prequant_out"]).reshape(nh, dk, dv).astype(np.float64)
    assert (np.sqrt(np.sum((R - ref["R"]) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
    if r > 0:
        p = host(st["comp_k"]).reshape(nh, r, dk).astype(np.float64)
        w = host(st["comp_v"]).reshape(nh, r, dv).astype(np.float64)
        C = np.einsum("hci,hcj->hij", p, w)
        Cr = np.einsum("hci,hcj->hij", ref["p"].astype(np.float64), ref["w"].astype(np.float64))
        assert (np.sqrt(np.sum((C - Cr) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
    # the flush's codes are the oracle's codec applied to its residual
    _assert_oracle_encoding(st, R, hp)


@pytest.mark.parametrize("name", ["gdn_serving", "kda", "damp"])
def test_window_free_running(name):
    """Four windows back to back on both sides.  Near-tie code flips make
    the quantized trajectories part by design, so the bar is statistical:
    the GPU's mean output error against the unquantized fp64 trajectory is
    within x[0.8, 1.25] of the oracle's own windowed-INT8 error, and far
    below the error of per-step INT8."""
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[name], B=1, H=4)
    nh, dk, dv, W, r = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"]
    bf = cfg["io"] == "bf16"
    hp = _hp_rows(cfg, nh) if cfg.get("n_hp") else None
    nwin = 4
    T = nwin * W
    S0 = _warm_state(cfg, nh)
    inp = synth.steps_inputs(cfg, 0, T)
    _, o_exact = oracle.recur(S0, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    enc = oracle.compress(S0.astype(np.float64), r, 20, hp_idx=hp)
    d = desc_for(cfg)
    st = g.alloc_state(d)
    _upload(torch, st, enc, hp)
    o_orc = np.empty((T, nh, dv))
    o_gpu = np.empty((T, nh, dv))
    say("free-running", name)
    for wi in range(nwin):
        sl = {k: v[wi * W:(wi + 1) * W] for k, v in inp.items()}
        o_ref, _, SW = oracle.window(_base(enc, hp), sl["q"], sl["k"], sl["v"], sl["a"], sl["b"])
        o_orc[wi * W:(wi + 1) * W] = o_ref
        enc = oracle.compress(SW, r, 20, hp_idx=hp)
        outs = _run_gpu_window(torch, g, d, st, sl, W, bf, torch.bfloat16 if bf else torch.float32)
        g.gdn_quant_window_flush(d, st, W)
        for t in range(W):
            o_gpu[wi * W + t] = host_io(outs[t], bf).reshape(nh, dv)
    err_gpu = np.mean([per_head_rel(o_gpu[t], o_exact[t]).mean() for t in range(T)])
    err_orc = np.mean([per_head_rel(o_orc[t], o_exact[t]).mean() for t in range(T)])
    floor = 2e-3 if bf else 0.0   # the GPU's bf16 output rounding adds this much at most
    assert err_gpu <= 1.25 * err_orc + floor and err_gpu >= 0.8 * err_orc, (err_gpu, err_orc)
    assert err_orc < 0.05


def test_per_step_damp_layout():
    """Per-step mode (W = 1, r = 0) with the DAMP layout runs the window step
    and a one-token flush inside gdn_quant_decode_step."""
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS["damp"], B=1, H=4, W=1, r=0)
    nh, dk, dv = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"]
    hp = _hp_rows(cfg, nh)
    d = desc_for(cfg, flags=g.DEBUG_PREQUANT)
    enc = oracle.compress(_warm_state(cfg, nh).astype(np.float64), 0, 20, hp_idx=hp)
    st = g.alloc_state(d)
    _upload(torch, st, enc, hp)
    inp = synth.steps_inputs(cfg, 0, 1)
    o = _run_gpu_window(torch, g, d, st, inp, 1, True, torch.bfloat16)[0]
    torch.cuda.synchronize()
    o_ref, _, SW = oracle.window(_base(enc, hp), inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    check_outputs(host_io(o, True), o_ref[0], True)
    R = host(st["prequant_out"]).reshape(nh, dk, dv)
    assert per_head_rel(R, SW).max() <= 1e-4
    _assert_oracle_encoding(st, R, hp)


def test_checkpoint_restore_and_determinism():
    """The state arrays are the checkpoint: copying them mid-window and
    continuing from the copy reproduces the uninterrupted run bit for bit,
    and two identical runs are bit-identical (no atomics anywhere)."""
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS["kda"], B=1, H=4, W=8, r=2)
    nh = cfg["B"] * cfg["H"]
    d = desc_for(cfg)
    S0 = _warm_state(cfg, nh)
    inp = synth.steps_inputs(cfg, 0, 8)

    def fresh():
        st = g.alloc_state(d)
        g.gdn_state_quantize(d, dev(S0), st)
        return st

    say("checkpoint")
    st_a = fresh()
    outs_a = _run_gpu_window(torch, g, d, st_a, inp, 8, True, torch.bfloat16)
    g.gdn_quant_window_flush(d, st_a, 8)
    st_b = fresh()
    first = {k: v[:3] for k, v in inp.items()}
    outs_b = _run_gpu_window(torch, g, d, st_b, first, 3, True, torch.bfloat16)
    snap = {k: (None if v is None else v.clone()) for k, v in st_b.items()}
    # scribble over the live state, then restore from the snapshot
    for v in st_b.values():
        if v is not None:
            v.fill_(7)
    for k, v in snap.items():
        if v is not None:
            st_b[k].copy_(v)
    for t in range(3, 8):
        o = torch.empty(nh * d.dv, dtype=torch.bfloat16, device="cuda")
        one = {k: v[t] for k, v in inp.items()}
        g.gdn_quant_decode_step(d, st_b, dev_io(one, "q", True), dev_io(one, "k", True),
                                dev_io(one, "v", True), dev(one["a"]), dev(one["b"]), o, t)
        outs_b.append(o)
    g.gdn_quant_window_flush(d, st_b, 8)
    torch.cuda.synchronize()
    for oa, ob in zip(outs_a, outs_b):
        assert torch.equal(oa.view(torch.int16), ob.view(torch.int16))
    for k in st_a:
        if st_a[k] is not None:
            assert torch.equal(st_a[k], st_b[k]), k


@pytest.mark.parametrize("case", [
    # the library's limits: window 256, 8 compensators, 64 DAMP rows
    dict(name="kda", over=dict(B=1, H=2, W=256, r=8), n=256, warm=48),
    dict(name="damp", over=dict(B=1, H=2, W=8, r=8, n_hp=64), n=8, warm=48),
    # the serving workload's own window start: 512 fp32 warm-up steps
    dict(name="gdn_serving", over=dict(B=1, H=3), n=16, warm=512),
], ids=["W256-r8", "r8-nhp64", "warmup512"])
def test_window_limits_and_warmup(case):
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[case["name"]], **case["over"])
    nh, dk, dv, W, r = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"]
    n = case["n"]
    hp = _hp_rows(cfg, nh) if cfg.get("n_hp") else None
    d = desc_for(cfg, flags=g.DEBUG_PREQUANT)
    enc = oracle.compress(_warm_state(cfg, nh, steps=case["warm"]).astype(np.float64), r, 20, hp_idx=hp)
    st = g.alloc_state(d)
    _upload(torch, st, enc, hp)
    inp = synth.steps_inputs(cfg, 0, n)
    say("limits", case)
    outs = _run_gpu_window(torch, g, d, st, inp, n, True, torch.bfloat16)
    g.gdn_quant_window_flush(d, st, n)
    torch.cuda.synchronize()
    o_ref, _, SW = oracle.window(_base(enc, hp), inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    for t in range(0, n, max(1, n // 16)):
        check_outputs(host_io(outs[t], True), o_ref[t], True)
    check_outputs(host_io(outs[n - 1], True), o_ref[n - 1], True)
    ref = oracle.compress(SW, r, 20, hp_idx=hp)
    scale = np.sqrt(np.sum(SW ** 2, axis=(1, 2)))
    R = host(st["prequant_out"]).reshape(nh, dk, dv).astype(np.float64)
    assert (np.sqrt(np.sum((R - ref["R"]) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
    _assert_oracle_encoding(st, R, hp)


@pytest.mark.parametrize("name,n", [("kda", None), ("kda", 11), ("gdn_serving", None), ("damp", None)])
def test_window_small_gates(name, n):
    """Gates far below the workloads' U[0.8, 1] (LinQuant Table 3 puts no
    bound on the gate): every gate log-uniform in [1e-3, 1], and per head a
    few channels (KDA) or steps (scalar gate) with a run of 1e-30 gates, one
    subnormal gate (1e-40) and a run of exact ones.  Over a whole window the
    gate products fall far below fp32's range (to about 1e-100) while the
    ratios between nearby tokens stay ordinary.  Outputs, buffered updates,
    the flush's residual, compensators and codes against the oracle, at the
    bars of the teacher-forced window test; a partial window too."""
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[name], B=1, H=3)
    nh, dk, dv, W, r = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"]
    n = n or W
    hp = _hp_rows(cfg, nh) if cfg.get("n_hp") else None
    d = desc_for(cfg, flags=g.DEBUG_PREQUANT)
    enc = oracle.compress(_warm_state(cfg, nh).astype(np.float64), r, 20, hp_idx=hp)
    st = g.alloc_state(d)
    _upload(torch, st, enc, hp)
    inp = synth.steps_inputs(cfg, 0, n)
    gr = synth.misc_rng(cfg["seed"], 41)
    a = (10.0 ** gr.uniform(-3.0, 0.0, inp["a"].shape)).astype(np.float32)   # [n, nh, 1|dk]
    width = a.shape[2]
    for h in range(nh):
        for j, ch in enumerate(gr.choice(width, min(3, width), replace=False)):
            t0 = int(gr.integers(0, max(1, n - 3)))
            if j == 0:
                a[t0:t0 + 2, h, ch] = np.float32(1e-30)
            elif j == 1:
                a[t0, h, ch] = np.float32(1e-40)          # an fp32 subnormal
            else:
                a[t0:t0 + 3, h, ch] = np.float32(1.0)
    assert (a > 0).all() and (a <= 1).all()
    inp["a"] = a
    bf = cfg["io"] == "bf16"
    say("window small gates", name, n)
    outs = _run_gpu_window(torch, g, d, st, inp, n, bf, torch.bfloat16 if bf else torch.float32)
    g.gdn_quant_window_flush(d, st, n)
    torch.cuda.synchronize()
    prod = np.prod(a.astype(np.float64), axis=0)
    assert prod.min() < 1e-60          # the products leave fp32's range
    o_ref, u_ref, SW = oracle.window(_base(enc, hp), inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    for t in range(n):
        check_outputs(host_io(outs[t], bf), o_ref[t], bf)
    u_gpu = host(st["buf_u"]).reshape(nh, W, dv)[:, :n].transpose(1, 0, 2)
    assert per_head_rel(u_gpu.reshape(n * nh, dv), u_ref.reshape(n * nh, dv)).max() <= 1e-4
    assert np.isfinite(host(st["buf_k"])).all()
    ref = oracle.compress(SW, r, 20, hp_idx=hp)
    scale = np.sqrt(np.sum(SW ** 2, axis=(1, 2)))
    R = host(st["prequant_out"]).reshape(nh, dk, dv).astype(np.float64)
    assert (np.sqrt(np.sum((R - ref["R"]) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
    if r > 0:
        p = host(st["comp_k"]).reshape(nh, r, dk).astype(np.float64)
        w = host(st["comp_v"]).reshape(nh, r, dv).astype(np.float64)
        C = np.einsum("hci,hcj->hij", p, w)
        Cr = np.einsum("hci,hcj->hij", ref["p"].astype(np.float64), ref["w"].astype(np.float64))
        assert (np.sqrt(np.sum((C - Cr) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
    _assert_oracle_encoding(st, R, hp)
