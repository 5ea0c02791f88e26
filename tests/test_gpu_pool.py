"""Serving shape through the C ABI: the pool entry points (state slots,
per-entry window positions and flush lengths, skipped entries) and shared
key heads (desc.hk < H).

Pool form against the oracle: entries on permuted slots (one slot out of
range, so skipped) run one per-step decode, and entries whose windows start
at different steps (so each call holds them at different positions, and an
entry before its start is skipped by its position) run to a flush that ends
every window with its own token count (partial windows, and one entry with
n_tokens = 0 left untouched).  Each active entry's outputs and buffered
updates meet the per-step and window bars against the oracle on that slot's
state, and the codes and scales the kernels store equal the oracle's codec
applied to the fp32 tensor they handed to it, bit for bit.

Pool form against the plain calls: every pool call is also compared bit for
bit with the plain calls on twin states (one plain state per entry, holding
a copy of that entry's slot): the same kernels run either way, so outputs,
codes, scales, compensators, buffers and gates must be identical; slots no
entry uses, and entries with an out-of-range slot, position or token count,
stay untouched.

Shared key heads: value head hh reads key head hh / (H / hk); the oracle is
run with q and k repeated over their value heads (plain data movement in the
test), with the parity bars of the per-step and window tests.
"""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu import (assert_encoding_is_oracle_codec, check_outputs, desc_for, dev, dev_io, host, host_io,
                        lib, per_head_rel, say, sub_cfg, torch_cuda)

pytestmark = pytest.mark.gpu

KEYS = ("codes", "row_scale", "col_scale", "comp_k", "comp_v", "buf_k", "buf_u", "buf_g", "g_cur", "hp_rows")


def _slot_view(st, name, slot, n_slots):
    t = st[name]
    per = t.numel() // n_slots
    return t[slot * per:(slot + 1) * per]


def _twin(torch, g, d1, pool_st, slot, n_slots):
    """A plain one-entry state holding a copy of one pool slot."""
    st = g.alloc_state(d1)
    for k in KEYS + ("hp_idx",):
        if pool_st.get(k) is not None and st.get(k) is not None:
            st[k].copy_(_slot_view(pool_st, k, slot, n_slots))
    return st


def _bytes_equal(a, b):
    torch = torch_cuda()
    return torch.equal(a.contiguous().view(torch.uint8), b.contiguous().view(torch.uint8))


def _inputs(torch, cfg, nb, t, bf):
    inp = synth.step_inputs(dict(cfg, B=nb), t)
    return inp, [dev_io(inp, "q", bf), dev_io(inp, "k", bf), dev_io(inp, "v", bf), dev(inp["a"]), dev(inp["b"])]


@pytest.mark.parametrize("bits", [8, 4])
def test_pool_per_step(bits):
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS["prefix_cache"], B=1, H=4)
    H, dk, dv = cfg["H"], cfg["dk"], cfg["dv"]
    n_slots = 7
    slots = [5, 0, 3, -1, 9]            # the last two are skipped
    nb = len(slots)
    d = desc_for(cfg, B=nb, W=1, r=0, bits=bits)
    dpool = desc_for(cfg, B=n_slots, W=1, r=0, bits=bits)
    d1 = desc_for(cfg, B=1, W=1, r=0, bits=bits)
    S = synth.prefill_states(dict(cfg, B=n_slots), heads=range(n_slots * H))
    pool = g.alloc_state(dpool)
    g.gdn_state_quantize(dpool, dev(S), pool)
    before = {k: pool[k].clone() for k in KEYS if pool.get(k) is not None}
    twins = {e: _twin(torch, g, d1, pool, s, n_slots) for e, s in enumerate(slots) if 0 <= s < n_slots}
    inp, args = _inputs(torch, cfg, nb, 0, True)
    o = torch.full((nb * H * dv,), 7.0, dtype=torch.bfloat16, device="cuda")
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    say("pool per-step", bits)
    g.gdn_quant_decode_step_pool(d, pool, n_slots, sl, None, *args, o)
    for e, st1 in twins.items():
        o1 = torch.empty(H * dv, dtype=torch.bfloat16, device="cuda")
        one = {k: v.reshape(nb, H, -1)[e] for k, v in inp.items()}
        g.gdn_quant_decode_step(d1, st1, dev_io(one, "q", True), dev_io(one, "k", True), dev_io(one, "v", True),
                                dev(one["a"]), dev(one["b"]), o1, 0)
        torch.cuda.synchronize()
        assert _bytes_equal(o.view(nb, H * dv)[e], o1), e
        for k in KEYS:
            if pool.get(k) is not None:
                assert _bytes_equal(_slot_view(pool, k, slots[e], n_slots), st1[k]), (e, k)
    torch.cuda.synchronize()
    used = {s for s in slots if 0 <= s < n_slots}
    for s in range(n_slots):
        if s not in used:
            for k in before:
                assert _bytes_equal(_slot_view(pool, k, s, n_slots), _slot_view(before, k, s, n_slots)), (s, k)
    for e, s in enumerate(slots):
        if not 0 <= s < n_slots:
            assert torch.all(o.view(nb, H * dv)[e] == 7.0)


def test_pool_window_positions_and_flush():
    """Three entries at different window positions in one call, then one
    flush call that ends two of the windows (n_tokens = position + 1) and
    leaves the third untouched (n_tokens = 0)."""
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS["gdn_serving"], B=1, H=3)
    H, dk, dv, W, r = cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"]
    n_slots = 6
    slots = [4, 1, 2]
    pos = [0, 5, 11]
    nb = len(slots)
    d = desc_for(cfg, B=nb)
    dpool = desc_for(cfg, B=n_slots)
    d1 = desc_for(cfg, B=1)
    S = synth.random_states(cfg["seed"], n_slots * H, dk, dv, scale=0.3)
    pool = g.alloc_state(dpool)
    g.gdn_state_quantize(dpool, dev(S), pool)
    twins = {e: _twin(torch, g, d1, pool, s, n_slots) for e, s in enumerate(slots)}
    say("pool window: history")
    # each entry's own history: pos[e] tokens through the pool API (one
    # entry per call) and through the plain API on its twin
    for e, s in enumerate(slots):
        for t in range(pos[e]):
            inp, args = _inputs(torch, cfg, 1, 100 * e + t, True)
            o = torch.empty(H * dv, dtype=torch.bfloat16, device="cuda")
            g.gdn_quant_decode_step_pool(desc_for(cfg, B=1), pool, n_slots,
                                         torch.tensor([s], dtype=torch.int32, device="cuda"),
                                         torch.tensor([t], dtype=torch.int32, device="cuda"), *args, o)
            g.gdn_quant_decode_step(d1, twins[e], *args, o, t)
    torch.cuda.synchronize()
    say("pool window: mixed positions")
    inp, args = _inputs(torch, cfg, nb, 999, True)
    o = torch.empty(nb * H * dv, dtype=torch.bfloat16, device="cuda")
    g.gdn_quant_decode_step_pool(d, pool, n_slots, torch.tensor(slots, dtype=torch.int32, device="cuda"),
                                 torch.tensor(pos, dtype=torch.int32, device="cuda"), *args, o)
    for e in range(nb):
        one = {k: v.reshape(nb, H, -1)[e] for k, v in inp.items()}
        o1 = torch.empty(H * dv, dtype=torch.bfloat16, device="cuda")
        g.gdn_quant_decode_step(d1, twins[e], dev_io(one, "q", True), dev_io(one, "k", True),
                                dev_io(one, "v", True), dev(one["a"]), dev(one["b"]), o1, pos[e])
        torch.cuda.synchronize()
        assert _bytes_equal(o.view(nb, H * dv)[e], o1), e
        for k in KEYS:
            if pool.get(k) is not None:
                assert _bytes_equal(_slot_view(pool, k, slots[e], n_slots), twins[e][k]), (e, k)
    say("pool window: flush")
    ntok = [pos[0] + 1, 0, pos[2] + 1]
    keep = {k: _slot_view(pool, k, slots[1], n_slots).clone() for k in KEYS if pool.get(k) is not None}
    g.gdn_quant_window_flush_pool(d, pool, n_slots, torch.tensor(slots, dtype=torch.int32, device="cuda"),
                                  torch.tensor(ntok, dtype=torch.int32, device="cuda"))
    for e in (0, 2):
        g.gdn_quant_window_flush(d1, twins[e], ntok[e])
    torch.cuda.synchronize()
    for e in (0, 2):
        for k in KEYS:
            if pool.get(k) is not None:
                assert _bytes_equal(_slot_view(pool, k, slots[e], n_slots), twins[e][k]), (e, k)
    for k, v in keep.items():
        assert _bytes_equal(_slot_view(pool, k, slots[1], n_slots), v), k


def _expand(x, H, hk):
    """[n, B*hk, d] key-head arrays -> [n, B*H, d]: value head hh reads key head hh // (H/hk)."""
    n, nk, dd = x.shape
    B = nk // hk
    idx = np.array([b * hk + hh // (H // hk) for b in range(B) for hh in range(H)])
    return x[:, idx]


@pytest.mark.parametrize("case", [("prefix_cache", dict(B=2, H=8), 2), ("tiny", dict(H=4), 1)],
                         ids=["prefix-hk2", "tiny-hk1"])
def test_shared_key_heads_per_step(case):
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[case[0]], **case[1])
    hk = case[2]
    B, H, dk, dv = cfg["B"], cfg["H"], cfg["dk"], cfg["dv"]
    nh = B * H
    bf = cfg["io"] == "bf16"
    d = desc_for(cfg, W=1, r=0, hk=hk, flags=g.DEBUG_PREQUANT)
    S = (synth.prefill_states(cfg, heads=range(nh)) if cfg.get("outlier_rows")
         else synth.random_states(12, nh, dk, dv) * np.float32(0.3))
    Q, s, c = oracle.quantize(S)
    st = g.alloc_state(d)
    st["codes"].copy_(torch.from_numpy(Q.reshape(-1)))
    st["row_scale"].copy_(torch.from_numpy(s.reshape(-1)))
    st["col_scale"].copy_(torch.from_numpy(c.reshape(-1)))
    inp = synth.step_inputs(dict(cfg, H=hk), 5)         # q, k: [B*hk, dk]
    vab = synth.step_inputs(cfg, 6)                     # v, a, b: per value head
    o = torch.empty(nh * dv, dtype=torch.bfloat16 if bf else torch.float32, device="cuda")
    say("shared key heads per-step", case)
    g.gdn_quant_decode_step(d, st, dev_io(inp, "q", bf), dev_io(inp, "k", bf), dev_io(vab, "v", bf),
                            dev(vab["a"]), dev(vab["b"]), o, 0)
    torch.cuda.synchronize()
    qx, kx = _expand(inp["q"][None], H, hk)[0], _expand(inp["k"][None], H, hk)[0]
    ref = oracle.quant_step(Q, s, c, qx, kx, vab["v"], vab["a"], vab["b"])
    check_outputs(host_io(o, bf), ref["o"], bf)
    assert per_head_rel(host(st["prequant_out"]).reshape(nh, dk, dv), ref["S_pre"]).max() <= 1e-4
    # the fp32-state kernel reads shared keys the same way
    Sd = dev(S)
    of = torch.empty_like(o)
    g.gdn_fp32_decode_step(d, Sd, dev_io(inp, "q", bf), dev_io(inp, "k", bf), dev_io(vab, "v", bf),
                           dev(vab["a"]), dev(vab["b"]), of)
    torch.cuda.synchronize()
    S_ref, o_ref = oracle.recur(S, qx[None], kx[None], vab["v"][None], vab["a"][None], vab["b"][None])
    check_outputs(host_io(of, bf), o_ref[0], bf)
    assert per_head_rel(host(Sd).reshape(nh, dk, dv), S_ref).max() <= 1e-5


def test_shared_key_heads_window():
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS["kda"], B=2, H=4)
    hk = 2
    B, H, dk, dv, W, r = cfg["B"], cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"]
    nh = B * H
    n = 6
    d = desc_for(cfg, hk=hk)
    S0 = synth.random_states(cfg["seed"], nh, dk, dv, scale=0.3).astype(np.float64)
    enc = oracle.compress(S0, r, 20)
    st = g.alloc_state(d)
    for k, v in (("codes", enc["Q"]), ("row_scale", enc["s"]), ("col_scale", enc["c"]),
                 ("comp_k", enc["p"]), ("comp_v", enc["w"])):
        st[k].copy_(torch.from_numpy(np.ascontiguousarray(v).reshape(-1)))
    kq = synth.steps_inputs(dict(cfg, H=hk), 0, n)
    vab = synth.steps_inputs(cfg, 50, n)
    outs = []
    say("shared key heads window")
    for t in range(n):
        o = torch.empty(nh * dv, dtype=torch.bfloat16, device="cuda")
        g.gdn_quant_decode_step(d, st, dev_io({"q16": kq["q16"][t]}, "q", True), dev_io({"k16": kq["k16"][t]}, "k", True),
                                dev_io({"v16": vab["v16"][t]}, "v", True), dev(vab["a"][t]), dev(vab["b"][t]), o, t)
        outs.append(o)
    torch.cuda.synchronize()
    X0 = oracle.state_base(enc["Q"], enc["s"], enc["c"], enc["p"], enc["w"])
    o_ref, _, _ = oracle.window(X0, _expand(kq["q"], H, hk), _expand(kq["k"], H, hk), vab["v"], vab["a"], vab["b"])
    for t in range(n):
        check_outputs(host_io(outs[t], True), o_ref[t], True)


def test_pool_per_step_static_scales():
    """Static scales through the pool entry point: the row and column scale
    arrays hold two planes ([scales of every slot][reciprocals of every
    slot]); the pool step on permuted and skipped slots equals the plain
    static step on twin states holding each slot's codes and both planes,
    bit for bit, and the scales are never rewritten."""
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS["prefix_cache"], B=1, H=4)
    H, dk, dv = cfg["H"], cfg["dk"], cfg["dv"]
    n_slots = 7
    slots = [5, 0, 3, -1, 9]
    nb = len(slots)
    F = g.STATIC_SCALES
    d = desc_for(cfg, B=nb, W=1, r=0, flags=F)
    dpool = desc_for(cfg, B=n_slots, W=1, r=0, flags=F)
    d1 = desc_for(cfg, B=1, W=1, r=0, flags=F)
    S = synth.prefill_states(dict(cfg, B=n_slots), heads=range(n_slots * H))
    cal = synth.steps_inputs(dict(cfg, B=n_slots), 300, 4)
    pool = g.alloc_state(dpool)
    say("pool static fit")
    g.calibrate_static_scales(dpool, dev(S), dev_io(cal, "q", True), dev_io(cal, "k", True), dev_io(cal, "v", True),
                              dev(cal["a"]), dev(cal["b"]), 4, pool)
    g.gdn_state_quantize(dpool, dev(S), pool)

    def planes(st, name, slot, n):
        t = st[name].view(2, n, -1)
        return t[0, slot], t[1, slot]

    twins = {}
    for e, s in enumerate(slots):
        if 0 <= s < n_slots:
            st = g.alloc_state(d1)
            st["codes"].copy_(_slot_view(pool, "codes", s, n_slots))
            for name in ("row_scale", "col_scale"):
                p0, p1 = planes(pool, name, s, n_slots)
                st[name].view(2, -1)[0].copy_(p0)
                st[name].view(2, -1)[1].copy_(p1)
            twins[e] = st
    scales = (pool["row_scale"].clone(), pool["col_scale"].clone())
    codes_before = pool["codes"].clone()
    inp, args = _inputs(torch, cfg, nb, 0, True)
    o = torch.full((nb * H * dv,), 7.0, dtype=torch.bfloat16, device="cuda")
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    say("pool static step")
    g.gdn_quant_decode_step_pool(d, pool, n_slots, sl, None, *args, o)
    for e, st1 in twins.items():
        o1 = torch.empty(H * dv, dtype=torch.bfloat16, device="cuda")
        one = {k: v.reshape(nb, H, -1)[e] for k, v in inp.items()}
        g.gdn_quant_decode_step(d1, st1, dev_io(one, "q", True), dev_io(one, "k", True), dev_io(one, "v", True),
                                dev(one["a"]), dev(one["b"]), o1, 0)
        torch.cuda.synchronize()
        assert _bytes_equal(o.view(nb, H * dv)[e], o1), e
        assert _bytes_equal(_slot_view(pool, "codes", slots[e], n_slots), st1["codes"]), e
    torch.cuda.synchronize()
    assert torch.equal(scales[0], pool["row_scale"]) and torch.equal(scales[1], pool["col_scale"])
    used = {s for s in slots if 0 <= s < n_slots}
    for s in range(n_slots):
        if s not in used:
            assert _bytes_equal(_slot_view(pool, "codes", s, n_slots), _slot_view({"codes": codes_before}, "codes", s,
                                                                                   n_slots)), s
    for e, s in enumerate(slots):
        if not 0 <= s < n_slots:
            assert torch.all(o.view(nb, H * dv)[e] == 7.0)


def _heads(slot, H):
    return np.arange(slot * H, (slot + 1) * H)


def test_pool_per_step_against_oracle():
    """Per-step decode through the pool entry point on permuted slots (one
    out of range), each active entry checked against the oracle's per-step
    decode of its slot's state: outputs, the pre-quantization state, and
    codes and scales bit for bit against the oracle's codec on the kernel's
    own input; slots no entry uses keep the oracle's encoding."""
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS["prefix_cache"], B=1, H=4)
    H, dk, dv = cfg["H"], cfg["dk"], cfg["dv"]
    n_slots = 6
    slots = [4, 1, -1, 3, 0]
    nb = len(slots)
    d = desc_for(cfg, B=nb, W=1, r=0, flags=g.DEBUG_PREQUANT)
    dpool = desc_for(cfg, B=n_slots, W=1, r=0, flags=g.DEBUG_PREQUANT)
    S = synth.prefill_states(dict(cfg, B=n_slots), heads=range(n_slots * H))
    Q, s_, c_ = oracle.quantize(S)
    pool = g.alloc_state(dpool)
    pool["codes"].copy_(torch.from_numpy(Q.reshape(-1)))
    pool["row_scale"].copy_(torch.from_numpy(s_.reshape(-1)))
    pool["col_scale"].copy_(torch.from_numpy(c_.reshape(-1)))
    inp, args = _inputs(torch, cfg, nb, 2, True)
    o = torch.full((nb * H * dv,), 7.0, dtype=torch.bfloat16, device="cuda")
    say("pool per-step vs oracle")
    g.gdn_quant_decode_step_pool(d, pool, n_slots, torch.tensor(slots, dtype=torch.int32, device="cuda"), None,
                                 *args, o)
    torch.cuda.synchronize()
    o_host = host_io(o, True).reshape(nb, H, dv)
    codes = host(pool["codes"]).reshape(n_slots * H, dk, dv)
    rs = host(pool["row_scale"]).reshape(n_slots * H, dk)
    cs = host(pool["col_scale"]).reshape(n_slots * H, dv)
    P = host(pool["prequant_out"]).reshape(n_slots * H, dk, dv)
    for e, slot in enumerate(slots):
        if not 0 <= slot < n_slots:
            assert np.all(o_host[e] == 7.0)
            continue
        hs, hi = _heads(slot, H), _heads(e, H)
        ref = oracle.quant_step(Q[hs], s_[hs], c_[hs], inp["q"][hi], inp["k"][hi], inp["v"][hi], inp["a"][hi],
                                inp["b"][hi])
        check_outputs(o_host[e], ref["o"], True)
        assert per_head_rel(P[hs], ref["S_pre"]).max() <= 1e-4
        assert_encoding_is_oracle_codec(P[hs], codes[hs], cs[hs], rs[hs])
    for slot in set(range(n_slots)) - set(slots):
        hs = _heads(slot, H)
        assert np.array_equal(codes[hs], Q[hs]) and np.array_equal(rs[hs], s_[hs])


@pytest.mark.parametrize("name", ["gdn_serving", "kda"])
def test_pool_window_staggered_against_oracle(name):
    """Window mode through the pool entry points with staggered windows:
    entry e starts its window at step start[e], so each decode call holds
    the entries at different positions (an entry before its start has
    position -1 and is skipped); one flush call then ends each window with
    its own token count W - start[e] (partial windows), skips an entry on
    an out-of-range slot, and leaves an entry with n_tokens = 0 untouched.
    Against the oracle's window decode and flush of each slot's tokens."""
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[name], B=1, H=2)
    H, dk, dv, W, r = cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"]
    n_slots = 6
    slots = [3, 0, 4, 9, 2]
    start = [0, 3, W // 2 - 1, 0, 5]
    ntok = [W - start[0], W - start[1], W - start[2], W, 0]
    nb = len(slots)
    d = desc_for(cfg, B=nb, flags=g.DEBUG_PREQUANT)
    dpool = desc_for(cfg, B=n_slots, flags=g.DEBUG_PREQUANT)
    S = synth.random_states(cfg["seed"] + 3, n_slots * H, dk, dv, scale=0.3).astype(np.float64)
    enc = oracle.compress(S, r, 20)
    pool = g.alloc_state(dpool)
    for k, v in (("codes", enc["Q"]), ("row_scale", enc["s"]), ("col_scale", enc["c"]), ("comp_k", enc["p"]),
                 ("comp_v", enc["w"])):
        pool[k].copy_(torch.from_numpy(np.ascontiguousarray(v).reshape(-1)))
    sl = torch.tensor(slots, dtype=torch.int32, device="cuda")
    steps = synth.steps_inputs(dict(cfg, B=nb), 0, W)
    outs = []
    say("pool window staggered", name)
    for i in range(W):
        one = {k: v[i] for k, v in steps.items()}
        pos = [i - start[e] if i >= start[e] else -1 for e in range(nb)]
        o = torch.full((nb * H * dv,), 7.0, dtype=torch.bfloat16, device="cuda")
        g.gdn_quant_decode_step_pool(d, pool, n_slots, sl, torch.tensor(pos, dtype=torch.int32, device="cuda"),
                                     dev_io(one, "q", True), dev_io(one, "k", True), dev_io(one, "v", True),
                                     dev(one["a"]), dev(one["b"]), o)
        outs.append(o)
    torch.cuda.synchronize()
    before = {k: host(pool[k]).copy() for k in KEYS if pool.get(k) is not None}
    say("pool flush staggered", name)
    g.gdn_quant_window_flush_pool(d, pool, n_slots, sl, torch.tensor(ntok, dtype=torch.int32, device="cuda"))
    torch.cuda.synchronize()
    o_all = np.stack([host_io(x, True).reshape(nb, H, dv) for x in outs])      # [W, nb, H, dv]
    u_all = host(pool["buf_u"]).reshape(n_slots * H, W, dv)
    P = host(pool["prequant_out"]).reshape(n_slots * H, dk, dv)
    after = {k: host(pool[k]) for k in before}
    for e, slot in enumerate(slots):
        if not 0 <= slot < n_slots:
            assert np.all(o_all[:, e] == 7.0)
            continue
        hs, hi = _heads(slot, H), _heads(e, H)
        assert np.all(o_all[:start[e], e] == 7.0)
        tk = slice(start[e], W)
        n = W - start[e]
        X0 = oracle.state_base(enc["Q"][hs], enc["s"][hs], enc["c"][hs], enc["p"][hs], enc["w"][hs])
        o_ref, u_ref, SW = oracle.window(X0, steps["q"][tk][:, hi], steps["k"][tk][:, hi], steps["v"][tk][:, hi],
                                         steps["a"][tk][:, hi], steps["b"][tk][:, hi])
        for t in range(n):
            check_outputs(o_all[start[e] + t, e], o_ref[t], True)
        u_gpu = u_all[hs][:, :n].transpose(1, 0, 2)
        assert per_head_rel(u_gpu.reshape(n * H, dv), u_ref.reshape(n * H, dv)).max() <= 1e-4
        if ntok[e] == 0:
            for k in before:      # not flushed: the whole slot is as the decode steps left it
                per = before[k].size // n_slots
                assert np.array_equal(after[k].reshape(-1)[slot * per:(slot + 1) * per],
                                      before[k].reshape(-1)[slot * per:(slot + 1) * per]), k
            continue
        ref = oracle.compress(SW, r, 20)
        scale = np.sqrt(np.sum(SW ** 2, axis=(1, 2)))
        R = P[hs].astype(np.float64)
        assert (np.sqrt(np.sum((R - ref["R"]) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
        pk = after["comp_k"].reshape(n_slots * H, r, dk)[hs].astype(np.float64)
        wv = after["comp_v"].reshape(n_slots * H, r, dv)[hs].astype(np.float64)
        C = np.einsum("hci,hcj->hij", pk, wv)
        Cr = np.einsum("hci,hcj->hij", ref["p"].astype(np.float64), ref["w"].astype(np.float64))
        assert (np.sqrt(np.sum((C - Cr) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
        assert_encoding_is_oracle_codec(P[hs], after["codes"].reshape(n_slots * H, dk, dv)[hs],
                                        after["col_scale"].reshape(n_slots * H, dv)[hs],
                                        after["row_scale"].reshape(n_slots * H, dk)[hs])
