"""Chunkwise prefill (gdn_prefill) through the C ABI against the oracle's
sequential recurrence (oracle.recur: the Gated DeltaNet and KDA rows of
LinQuant's Table 3 run token by token in fp64).

The kernels compute the same recurrence 32 tokens (scalar gate, D = 128),
64 tokens (scalar gate, D = 64) or 16 tokens (per-channel gate) at a time with bf16 matrix products whose fp32
operands are split in two bf16 parts (operand error near 2^-17), so the
bars are those of fp32 arithmetic on bf16 inputs:
  * state after the last token: l2-relative error per head <= 1e-4;
  * outputs (bf16): every element is a correct bf16 rounding of a value
    within 1e-4 of its token's largest |o| of the oracle, and per head the
    l2 gap to the oracle's output rounded to bf16 is <= 2e-3 of its norm.
Cases, for both gates: several chunks with a ragged tail, one partial
chunk, one token, exact chunk multiples, both head sizes, shared key heads,
the identity gates (a = 1, b = 0 keep the state bit for bit), sampled heads
of the full-size workloads; and T = 0, prefill followed by
gdn_state_quantize, a per-channel gate whose channels are all equal (the
scalar-gate kernel's result within the bars), and gates small enough that
a chunk's decay underflows (either gate).
"""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu import bf16_half_ulp, desc_for, dev, host, lib, per_head_rel, say, torch_cuda

pytestmark = pytest.mark.gpu


def _cfg(B, H, D, seed, decay="scalar"):
    return dict(B=B, H=H, dk=D, dv=D, io="bf16", decay=decay, a_lo=0.90 if decay == "scalar" else 0.80, W=1, r=0,
                seed=seed)


def _inputs(cfg, T, hk=None):
    """Token-major inputs [B,T,H,.] (and [B,T,hk,dk] for q, k) plus the
    oracle's [T, B*H, .] view with q, k repeated over their value heads."""
    B, H, D = cfg["B"], cfg["H"], cfg["dk"]
    hk = hk or H
    G = H // hk
    inp = synth.steps_inputs(cfg, 0, T)        # [T, B*H, ...]

    def bt(x):                                 # [T, B*H, ...] -> [B, T, H, ...]
        x = x.reshape((T, B, H) + x.shape[2:])
        return np.ascontiguousarray(np.swapaxes(x, 0, 1))

    out = {}
    for name in ("q", "k"):
        full = bt(inp[name + "16"])[:, :, ::G]          # key head kh = value head kh*G's draw
        out[name + "16"] = np.ascontiguousarray(full)
        rep = np.repeat(bt(inp[name])[:, :, ::G], G, axis=2)   # oracle: value head hh reads key hh // G
        out[name] = np.ascontiguousarray(np.swapaxes(rep, 0, 1).reshape(T, B * H, D))
    out["v16"] = bt(inp["v16"])
    out["v"] = inp["v"]
    out["a_dev"] = bt(inp["a"][..., 0] if cfg["decay"] == "scalar" else inp["a"])
    out["b_dev"] = bt(inp["b"])
    out["a"], out["b"] = inp["a"], inp["b"]
    return out


def _bf16_dev(bits):
    torch = torch_cuda()
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)


def _run(cfg, T, S0, hk=None):
    torch = torch_cuda()
    g = lib()
    B, H, D = cfg["B"], cfg["H"], cfg["dk"]
    inp = _inputs(cfg, T, hk)
    d = desc_for(cfg, hk=hk or 0)
    S = dev(S0.copy())
    o = torch.full((B, T, H, D), 3.0, dtype=torch.bfloat16, device="cuda")
    say("prefill", cfg["decay"], f"B={B} H={H} D={D} T={T} hk={hk}")
    g.gdn_prefill(d, S, _bf16_dev(inp["q16"]), _bf16_dev(inp["k16"]), _bf16_dev(inp["v16"]), dev(inp["a_dev"]),
                  dev(inp["b_dev"]), o, T)
    torch.cuda.synchronize()
    o_host = synth.bf16_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16))
    return inp, host(S), o_host


def _check(cfg, T, inp, S_got, o_got, S0, heads=None):
    """Compare with the oracle on all heads, or on the listed heads."""
    B, H, D = cfg["B"], cfg["H"], cfg["dk"]
    sel = np.arange(B * H) if heads is None else np.asarray(heads)
    S_ref, o_ref = oracle.recur(S0[sel], inp["q"][:, sel], inp["k"][:, sel], inp["v"][:, sel], inp["a"][:, sel],
                                inp["b"][:, sel])
    rel_S = per_head_rel(S_got.reshape(B * H, D, D)[sel], S_ref)
    assert rel_S.max() <= 1e-4, rel_S.max()
    got = np.swapaxes(o_got, 0, 1).reshape(T, B * H, D)[:, sel].astype(np.float64)   # [T, nh, D]
    rowmax = np.abs(o_ref).max(axis=2, keepdims=True)
    bound = bf16_half_ulp(np.maximum(np.abs(o_ref), np.abs(got))) + 1e-4 * rowmax
    bad = np.abs(got - o_ref) > bound
    assert not bad.any(), f"{bad.sum()} outputs off (worst {np.abs(got - o_ref).max()})"
    ref16 = synth.bf16_to_f32(synth.bf16_bits(o_ref.astype(np.float32))).astype(np.float64)
    like = np.sqrt(((got - ref16) ** 2).sum(axis=(0, 2))) / np.maximum(np.sqrt((o_ref ** 2).sum(axis=(0, 2))), 1e-300)
    assert like.max() <= 2e-3, like.max()
    return rel_S.max(), like.max()


DECAYS = ["scalar", "channel"]


@pytest.mark.parametrize("decay", DECAYS)
@pytest.mark.parametrize("D,T", [(128, 150), (128, 65), (128, 64), (128, 37), (128, 32), (128, 16), (128, 1), (64, 200), (64, 128),
                                 (64, 9)])
def test_prefill_parity(D, T, decay):
    cfg = _cfg(2, 3, D, seed=21 + T, decay=decay)
    S0 = synth.random_states(5 + T, cfg["B"] * cfg["H"], D, D, scale=0.5)
    inp, S, o = _run(cfg, T, S0)
    _check(cfg, T, inp, S, o, S0)


@pytest.mark.parametrize("decay", DECAYS)
def test_prefill_zero_state_long(decay):
    cfg = _cfg(1, 2, 128, seed=31, decay=decay)
    T = 700
    S0 = np.zeros((2, 128, 128), np.float32)
    inp, S, o = _run(cfg, T, S0)
    _check(cfg, T, inp, S, o, S0)


@pytest.mark.parametrize("decay", DECAYS)
def test_prefill_shared_key_heads(decay):
    cfg = _cfg(2, 4, 128, seed=41, decay=decay)
    T = 100
    S0 = synth.random_states(7, 8, 128, 128, scale=0.5)
    inp, S, o = _run(cfg, T, S0, hk=2)
    _check(cfg, T, inp, S, o, S0)


def test_prefill_equal_channel_gates_match_scalar_gate():
    """A per-channel gate whose channels are all equal is the scalar gate:
    the KDA kernel's result meets the oracle's scalar-gate bars too."""
    cfg = _cfg(1, 3, 128, seed=43)
    T = 90
    S0 = synth.random_states(17, 3, 128, 128, scale=0.5)
    inp = _inputs(cfg, T)
    kcfg = dict(cfg, decay="channel")
    kin = dict(inp, a_dev=np.ascontiguousarray(np.repeat(inp["a_dev"][..., None], 128, axis=3)))
    torch = torch_cuda()
    g = lib()
    S = dev(S0.copy())
    o = torch.empty((1, T, 3, 128), dtype=torch.bfloat16, device="cuda")
    say("prefill equal channel gates")
    g.gdn_prefill(desc_for(kcfg), S, _bf16_dev(kin["q16"]), _bf16_dev(kin["k16"]), _bf16_dev(kin["v16"]),
                  dev(kin["a_dev"]), dev(kin["b_dev"]), o, T)
    torch.cuda.synchronize()
    o_host = synth.bf16_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16))
    _check(cfg, T, inp, host(S), o_host, S0)


def test_prefill_kda_underflowing_gates():
    """Per-channel gates down to 1e-4: a 16-token chunk's decay reaches
    1e-64 (below fp32's range) in some channels; the kernel takes only
    non-positive exponents, so it neither overflows nor loses the state."""
    cfg = _cfg(1, 2, 128, seed=47, decay="channel")
    T = 80
    S0 = synth.random_states(19, 2, 128, 128, scale=0.5)
    inp = _inputs(cfg, T)
    rng = synth.misc_rng(47, 1)
    small = rng.uniform(1e-4, 1.0, inp["a"].shape).astype(np.float32)
    mask = rng.uniform(size=inp["a"].shape) < 0.1        # one channel in ten decays fast
    inp["a"] = np.where(mask, small, inp["a"]).astype(np.float32)
    inp["a_dev"] = np.ascontiguousarray(np.swapaxes(inp["a"].reshape(T, 1, 2, 128), 0, 1))
    torch = torch_cuda()
    g = lib()
    S = dev(S0.copy())
    o = torch.empty((1, T, 2, 128), dtype=torch.bfloat16, device="cuda")
    say("prefill kda small gates")
    g.gdn_prefill(desc_for(cfg), S, _bf16_dev(inp["q16"]), _bf16_dev(inp["k16"]), _bf16_dev(inp["v16"]),
                  dev(inp["a_dev"]), dev(inp["b_dev"]), o, T)
    torch.cuda.synchronize()
    o_host = synth.bf16_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.isfinite(host(S)).all()
    _check(cfg, T, inp, host(S), o_host, S0)


def test_prefill_underflowing_scalar_gates():
    """Scalar gates small enough that a 32-token chunk's decay leaves fp32's
    range: head 0 has eight gates of 1e-6 in a row inside its second chunk
    (a decay near 2^-160, so 2^g of the chunk's later tokens and
    2^(g_C - g) of its earlier ones flush to zero), head 1 a gate drawn from
    U[1e-4, 1] at one token in ten; T = 100 leaves a ragged last chunk."""
    cfg = _cfg(1, 2, 128, seed=49)
    T = 100
    S0 = synth.random_states(21, 2, 128, 128, scale=0.5)
    inp = _inputs(cfg, T)
    a = inp["a"].copy()                                   # [T, B*H, 1]
    a[40:48, 0, 0] = 1e-6
    rng = synth.misc_rng(49, 1)
    small = rng.uniform(1e-4, 1.0, T).astype(np.float32)
    pick = rng.uniform(size=T) < 0.1
    a[pick, 1, 0] = small[pick]
    inp["a"] = a
    inp["a_dev"] = np.ascontiguousarray(np.swapaxes(a[..., 0].reshape(T, 1, 2), 0, 1))
    torch = torch_cuda()
    g = lib()
    S = dev(S0.copy())
    o = torch.empty((1, T, 2, 128), dtype=torch.bfloat16, device="cuda")
    say("prefill scalar small gates")
    g.gdn_prefill(desc_for(cfg), S, _bf16_dev(inp["q16"]), _bf16_dev(inp["k16"]), _bf16_dev(inp["v16"]),
                  dev(inp["a_dev"]), dev(inp["b_dev"]), o, T)
    torch.cuda.synchronize()
    o_host = synth.bf16_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.isfinite(host(S)).all()
    _check(cfg, T, inp, host(S), o_host, S0)


def test_prefill_kda_chunk_paths():
    """A chunk whose decay in some channel passes 2^-60 takes the pairwise
    Gram sums, every other chunk the factored ones: chunk 1 of head 0 decays
    by about 2^-70 in channel 5 (three gates of 1e-7), chunk 2 of head 1 by
    about 2^-59.8 in channel 100 (two gates of 1e-9, the chunk's others 1:
    just inside the factored range, where its factors reach 2^+-59.8), and
    chunk 0 of head 2 by about 2^-70 in channel 7 (the first chunk's flag is
    set while the kernel's tables are first cleared); all heads in one
    call."""
    cfg = _cfg(1, 3, 128, seed=53, decay="channel")
    T = 80
    S0 = synth.random_states(23, 3, 128, 128, scale=0.5)
    inp = _inputs(cfg, T)
    a = inp["a"].copy()                                   # [T, B*H, dk]
    a[17:20, 0, 5] = 1e-7
    a[32:48, 1, 100] = 1.0
    a[40:42, 1, 100] = 1e-9
    a[2:5, 2, 7] = 1e-7
    inp["a"] = a
    inp["a_dev"] = np.ascontiguousarray(np.swapaxes(a.reshape(T, 1, 3, 128), 0, 1))
    torch = torch_cuda()
    g = lib()
    S = dev(S0.copy())
    o = torch.empty((1, T, 3, 128), dtype=torch.bfloat16, device="cuda")
    say("prefill kda chunk paths")
    g.gdn_prefill(desc_for(cfg), S, _bf16_dev(inp["q16"]), _bf16_dev(inp["k16"]), _bf16_dev(inp["v16"]),
                  dev(inp["a_dev"]), dev(inp["b_dev"]), o, T)
    torch.cuda.synchronize()
    o_host = synth.bf16_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16))
    assert np.isfinite(host(S)).all()
    _check(cfg, T, inp, host(S), o_host, S0)


@pytest.mark.parametrize("decay", DECAYS)
@pytest.mark.parametrize("part", ["quarter", "half", "half+1"])
def test_prefill_heads_per_cu_splits(part, decay):
    """With fewer heads than CUs, dk = 128 splits each head's value columns
    over 4 (heads <= CUs/4) or 2 (heads <= CUs/2) workgroups, each redoing
    the chunk-local work: head counts on both sides of those lines, against
    the oracle, for both gates."""
    torch = torch_cuda()
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    H = {"quarter": ncu // 4, "half": ncu // 2, "half+1": ncu // 2 + 1}[part]
    cfg = _cfg(1, H, 128, seed=57, decay=decay)
    T = 40
    S0 = synth.random_states(27, H, 128, 128, scale=0.5)
    inp, S, o = _run(cfg, T, S0)
    _check(cfg, T, inp, S, o, S0)


def test_prefill_empty_is_noop():
    torch = torch_cuda()
    g = lib()
    cfg = _cfg(1, 2, 128, seed=51)
    S0 = synth.random_states(9, 2, 128, 128)
    S = dev(S0.copy())
    say("prefill T=0")
    g.gdn_prefill(desc_for(cfg), S, None, None, None, None, None, None, 0)
    torch.cuda.synchronize()
    assert np.array_equal(host(S), S0)


@pytest.mark.parametrize("decay", DECAYS)
def test_prefill_identity_gates_keep_state(decay):
    """a = 1, b = 0: every update is zero and the decay is e^0 = 1, so the
    state comes back bit for bit (outputs still checked against the oracle)."""
    torch = torch_cuda()
    g = lib()
    cfg = _cfg(1, 2, 128, seed=61, decay=decay)
    T = 90
    S0 = synth.random_states(11, 2, 128, 128)
    inp = _inputs(cfg, T)
    inp["a_dev"][:] = 1.0
    inp["b_dev"][:] = 0.0
    inp["a"][:] = 1.0
    inp["b"][:] = 0.0
    S = dev(S0.copy())
    o = torch.empty((1, T, 2, 128), dtype=torch.bfloat16, device="cuda")
    say("prefill identity gates")
    g.gdn_prefill(desc_for(cfg), S, _bf16_dev(inp["q16"]), _bf16_dev(inp["k16"]), _bf16_dev(inp["v16"]),
                  dev(inp["a_dev"]), dev(inp["b_dev"]), o, T)
    torch.cuda.synchronize()
    assert np.array_equal(host(S), S0)
    o_host = synth.bf16_to_f32(o.view(torch.int16).cpu().numpy().view(np.uint16))
    _check(cfg, T, inp, host(S), o_host, S0)


def test_prefill_then_quantize():
    """Prefill, then gdn_state_quantize: the codes are the oracle codec's on
    the prefilled fp32 state, and the dequantized state is the oracle's state
    within the codec's half-step bound plus the prefill's own error."""
    torch = torch_cuda()
    g = lib()
    cfg = _cfg(1, 4, 128, seed=71)
    T = 130
    S0 = synth.random_states(13, 4, 128, 128, scale=0.5)
    inp, S, o = _run(cfg, T, S0)
    d = desc_for(cfg)
    st = g.alloc_state(d)
    say("prefill then quantize")
    g.gdn_state_quantize(d, dev(S), st)
    torch.cuda.synchronize()
    Q, s, c = oracle.quantize(S.reshape(4, 128, 128))
    assert np.array_equal(host(st["codes"]).reshape(Q.shape), Q)
    assert np.array_equal(host(st["row_scale"]).reshape(s.shape), s)
    assert np.array_equal(host(st["col_scale"]).reshape(c.shape), c)
    S_ref, _ = oracle.recur(S0, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"])
    Xq = oracle.dequantize(Q, s, c).astype(np.float64)
    half = 0.5 * s.astype(np.float64)[:, :, None] * c.astype(np.float64)[:, None, :] * (1 + 2.0 ** -22)
    assert np.all(np.abs(Xq - S_ref) <= half + 1e-4 * np.abs(S_ref).max(axis=(1, 2), keepdims=True))


@pytest.mark.parametrize("D", [128, 64])
def test_prefill_rejects(D):
    torch = torch_cuda()
    g = lib()
    cfg = _cfg(1, 2, D, seed=81)
    S = torch.zeros((2, D, D), device="cuda")
    x = torch.zeros((1, 8, 2, D), dtype=torch.bfloat16, device="cuda")
    ab = torch.ones((1, 8, 2), device="cuda")
    for over, msg in ((dict(io_dtype=g.IO_F32), "bf16"), (dict(dv=64 if D == 128 else 128), "dk == dv")):
        with pytest.raises(g.GdnqError, match=msg):
            g.gdn_prefill(desc_for(cfg, **over), S, x, x, x, ab, ab, x.clone(), 8)


@pytest.mark.parametrize("wl", ["prefill", "prefill_kda"])
def test_prefill_full_size_sampled(wl):
    """The benchmark's workloads (8 sequences x 32 heads x 4096 tokens, zero
    initial state, scalar or per-channel gate) in the benchmark's launch,
    checked on sampled heads against the oracle's 4096-step recurrence."""
    torch = torch_cuda()
    g = lib()
    cfg = synth.WORKLOADS[wl]
    B, H, D, T = cfg["B"], cfg["H"], cfg["dk"], cfg["T"]
    x = synth.token_major_inputs(cfg, T)
    S = torch.zeros((B * H, D, D), dtype=torch.float32, device="cuda")
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    say("prefill full size", wl, B, H, T)
    g.gdn_prefill(desc_for(dict(cfg, W=1, r=0)), S, _bf16_dev(x["q16"]), _bf16_dev(x["k16"]), _bf16_dev(x["v16"]),
                  dev(x["a"]), dev(x["b"]), o, T)
    torch.cuda.synchronize()
    S_got = host(S)
    for b, h in ((0, 0), (3, 17), (7, 31)):
        f = lambda name: np.ascontiguousarray(synth.bf16_to_f32(x[name][b, :, h])[:, None, :])
        ga = x["a"][b, :, h, None, None] if cfg["decay"] == "scalar" else x["a"][b, :, h, None, :]
        S_ref, o_ref = oracle.recur(np.zeros((1, D, D), np.float32), f("q16"), f("k16"), f("v16"),
                                    np.ascontiguousarray(ga), x["b"][b, :, h, None])
        rel_S = per_head_rel(S_got[b * H + h][None], S_ref)
        assert rel_S.max() <= 1e-4, (b, h, rel_S.max())
        got = synth.bf16_to_f32(o[b, :, h].view(torch.int16).cpu().numpy().view(np.uint16)).astype(np.float64)
        ref = o_ref[:, 0]
        rowmax = np.abs(ref).max(axis=1, keepdims=True)
        bound = bf16_half_ulp(np.maximum(np.abs(ref), np.abs(got))) + 1e-4 * rowmax
        assert not (np.abs(got - ref) > bound).any(), (b, h, np.abs(got - ref).max())
