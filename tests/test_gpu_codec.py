"""GPU parity of the state codec (gdn_state_quantize / gdn_state_dequantize)
against the oracle, through the C ABI.

Bar: identical seeded fp32 input -> bit-identical codes, row scales,
column scales and fp16 rows (layout 0 and DAMP layout 1); dequantized
states bit-identical (two rounded fp32 products).  With Compensator Tokens
the compensators are floating point: their products must match to 1e-4 of
the state norm, and the codes must equal the GPU codec's own codes on the
residual the kernel handed to it (which the r = 0 case pins to the oracle
bit for bit).
"""
import numpy as np
import pytest

import oracle
import synth
from tests._gpu import assert_encoding_is_oracle_codec, dev, desc_for, host, lib, per_head_rel, say, sub_cfg, torch_cuda

pytestmark = pytest.mark.gpu


def _uneven(seed, nh, dk, dv):
    X = synth.random_states(seed, nh, dk, dv)
    g = synth.misc_rng(seed, 9)
    X *= (2.0 ** g.uniform(-8, 8, (nh, dk, 1))).astype(np.float32)
    X *= (2.0 ** g.uniform(-4, 4, (nh, 1, dv))).astype(np.float32)
    return X


def _ties(seed, nh, dk, dv):
    # Every row holds 4 (row scale 2, reciprocal 1/2 exactly) and column
    # maxima 2*127/64 (column reciprocal 64 exactly), so entries 2*(n+1/2)/64
    # land exactly on half-integers: round-half-even is exercised everywhere.
    g = synth.misc_rng(seed, 3)
    X = (2.0 * (g.integers(-127, 127, (nh, dk, dv)) + 0.5) / 64.0)
    X[:, :, 0] = 4.0
    X[:, 0, 1:] = 2.0 * 127 / 64
    return X.astype(np.float32)


def _edge(seed, nh, dk, dv):
    X = _uneven(seed, nh, dk, dv)
    X[0] = 0                                   # zero head
    X[1, 3, :] = 0                             # zero row
    X[1, :, 7] = 0                             # zero column
    X[2] *= np.float32(2.0 ** -140)            # subnormal head
    X[3, 5, :] *= np.float32(1e30)             # huge row
    X[4, :, 9] = np.float32(1e-44)             # reciprocal-overflow column
    X[5] = np.sign(X[5]) * np.float32(3.0e38)  # near fp32 max
    return X


def _codec_case(torch, g, nh, dk, dv, X, layout=0, hp=None):
    cfg = dict(B=1, H=nh, dk=dk, dv=dv, W=1, r=0, decay="scalar", io="f32")
    d = desc_for(cfg)
    if layout == 1:
        d.layout, d.n_hp = g.LAYOUT_DAMP, hp.shape[1]
    st = g.alloc_state(d)
    if layout == 1:
        st["hp_idx"].copy_(torch.from_numpy(hp.reshape(-1)))
    Xd = dev(X)
    say("codec", nh, dk, dv, "layout", layout)
    g.gdn_state_quantize(d, Xd, st)
    back = torch.empty_like(Xd)
    g.gdn_state_dequantize(d, st, back)
    torch.cuda.synchronize()
    return d, st, host(back)


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64), (128, 64), (64, 128)])
@pytest.mark.parametrize("kind", ["uneven", "ties", "edge", "prefill"])
def test_codec_bit_exact(dk, dv, kind):
    torch = torch_cuda()
    g = lib()
    nh = 9
    if kind == "uneven":
        X = _uneven(1, nh, dk, dv)
    elif kind == "ties":
        X = _ties(2, nh, dk, dv)
    elif kind == "edge":
        X = _edge(3, nh, dk, dv)
    else:
        cfg = sub_cfg(synth.WORKLOADS["prefix_cache"], dk=dk, dv=dv)
        X = synth.prefill_states(cfg, heads=range(nh))
    d, st, back = _codec_case(torch, g, nh, dk, dv, X)
    Q, s, c = oracle.quantize(X)
    gQ = host(st["codes"]).reshape(nh, dk, dv)
    assert np.array_equal(gQ, Q), f"{np.sum(gQ != Q)} codes differ"
    assert np.array_equal(host(st["row_scale"]).reshape(nh, dk), s)
    assert np.array_equal(host(st["col_scale"]).reshape(nh, dv), c)
    assert np.array_equal(back, oracle.dequantize(Q, s, c))


@pytest.mark.parametrize("dk,dv", [(128, 128), (64, 64)])
def test_damp_codec_bit_exact(dk, dv):
    torch = torch_cuda()
    g = lib()
    nh, n_hp = 7, 8
    X = _uneven(4, nh, dk, dv)
    X[2, :, 3] = 0
    X[3, 1, :] = np.float32(70000.0)           # saturating fp16 row if chosen
    gr = synth.misc_rng(4, 2)
    hp = np.stack([np.sort(gr.choice(dk, n_hp, replace=False)) for _ in range(nh)]).astype(np.int32)
    others = np.setdiff1d(np.arange(dk), [1])
    hp[3] = np.sort(np.concatenate([[1], gr.choice(others, n_hp - 1, replace=False)]))
    d, st, back = _codec_case(torch, g, nh, dk, dv, X, layout=1, hp=hp)
    Qc, c, rows = oracle.quantize_damp(X, hp)
    assert np.array_equal(host(st["codes"]).reshape(nh, dk - n_hp, dv), Qc)
    assert np.array_equal(host(st["col_scale"]).reshape(nh, dv), c)
    assert np.array_equal(host(st["hp_rows"]).view(np.uint16).reshape(nh, n_hp, dv), rows)
    assert np.array_equal(back, oracle.dequantize_damp(Qc, c, rows, hp))


@pytest.mark.parametrize("dk,n_hp", [(128, 8), (128, 64), (64, 32), (64, 3)])
def test_damp_codec_row_lists_at_word_edges(dk, n_hp):
    """The fp16-row lists the kernels turn into a per-32-row bit mask: rows at
    the edges of the mask words, whole words listed, the first and last rows,
    and the largest list a head may carry; codes, scales and rows against
    the oracle bit for bit."""
    torch = torch_cuda()
    g = lib()
    dv = dk
    gr = synth.misc_rng(17, n_hp)
    edges = [0, 31, 32, 63, 64, 95, 96, 127]
    lists = [
        [i for i in edges if i < dk],            # word edges (padded below)
        list(range(n_hp)),                        # the first rows
        list(range(dk - n_hp, dk)),               # the last rows
        list(range(0, dk, dk // n_hp))[:n_hp],    # spread evenly
        list(gr.choice(dk, n_hp, replace=False)), # anywhere
    ]
    hp = []
    for rows in lists:
        rows = sorted(set(rows))[:n_hp]
        rest = [i for i in range(dk) if i not in rows]
        rows = rows + list(gr.choice(rest, n_hp - len(rows), replace=False))
        hp.append(np.sort(np.array(rows)))
    hp = np.stack(hp).astype(np.int32)
    nh = hp.shape[0]
    X = _uneven(19, nh, dk, dv)
    d, st, back = _codec_case(torch, g, nh, dk, dv, X, layout=1, hp=hp)
    Qc, c, rows = oracle.quantize_damp(X, hp)
    assert np.array_equal(host(st["codes"]).reshape(nh, dk - n_hp, dv), Qc)
    assert np.array_equal(host(st["col_scale"]).reshape(nh, dv), c)
    assert np.array_equal(host(st["hp_rows"]).view(np.uint16).reshape(nh, n_hp, dv), rows)
    assert np.array_equal(back, oracle.dequantize_damp(Qc, c, rows, hp))


@pytest.mark.parametrize("layout", [0, 1])
@pytest.mark.parametrize("r", [1, 2, 4])
def test_codec_with_compensators(layout, r):
    torch = torch_cuda()
    g = lib()
    nh, dk, dv, n_hp = 12, 128, 128, 8
    X = _uneven(5, nh, dk, dv) * np.float32(0.01)
    # plant outlier rows / columns so the compensators have work to do
    cfg = synth.WORKLOADS["prefix_cache"]
    X += np.float32(0.2) * synth.prefill_states(cfg, heads=range(nh)) / np.float32(50)
    cfgc = dict(B=1, H=nh, dk=dk, dv=dv, W=16, r=r, decay="scalar", io="f32")
    d = desc_for(cfgc, flags=g.DEBUG_PREQUANT)
    hp = None
    if layout == 1:
        gr = synth.misc_rng(5, 2)
        hp = np.stack([np.sort(gr.choice(dk, n_hp, replace=False)) for _ in range(nh)]).astype(np.int32)
        d.layout, d.n_hp = g.LAYOUT_DAMP, n_hp
    st = g.alloc_state(d)
    if hp is not None:
        st["hp_idx"].copy_(torch.from_numpy(hp.reshape(-1)))
    say("codec+comp", r, layout)
    g.gdn_state_quantize(d, dev(X), st)
    torch.cuda.synchronize()
    ref = oracle.compress(X.astype(np.float64), r, 20, hp_idx=hp)
    p, w = host(st["comp_k"]).reshape(nh, r, dk), host(st["comp_v"]).reshape(nh, r, dv)
    C = np.einsum("hci,hcj->hij", p.astype(np.float64), w.astype(np.float64))
    Cref = np.einsum("hci,hcj->hij", ref["p"].astype(np.float64), ref["w"].astype(np.float64))
    scale = np.sqrt(np.sum(X.astype(np.float64) ** 2, axis=(1, 2)))
    err = np.sqrt(np.sum((C - Cref) ** 2, axis=(1, 2))) / scale
    assert err.max() <= 1e-4, err
    R = host(st["prequant_out"]).reshape(nh, dk, dv)
    assert (np.sqrt(np.sum((R - ref["R"]) ** 2, axis=(1, 2))) / scale).max() <= 1e-4
    # the codes are the oracle's codec applied to the kernel's residual R
    assert_encoding_is_oracle_codec(R, host(st["codes"]), host(st["col_scale"]),
                                    None if hp is not None else host(st["row_scale"]), hp_idx=hp,
                                    hp_rows=None if hp is None else host(st["hp_rows"]))
    # dequantize = D(Q) + compensators rebuilds X within the codec bound
    back = torch.empty((nh * dk * dv,), dtype=torch.float32, device="cuda")
    g.gdn_state_dequantize(d, st, back)
    torch.cuda.synchronize()
    rec = host(back).reshape(nh, dk, dv)
    assert per_head_rel(rec, X).max() < 0.02


def test_compensator_restart_path():
    """Columns come in exact +-pairs (column 2m+1 = -column 2m) of signed
    powers of two, so the all-equal start vector is annihilated exactly on
    both sides: the first power-iteration step returns zero and the
    iteration restarts from the largest column (ties between a pair go to
    the lower index).  Only the first compensator is compared: after
    deflation the entries are no longer powers of two, the oracle's exact
    fp64 cancellation restarts again while the GPU's fused multiply-adds
    leave a rounding-size start, and without a wide spectral gap 20 steps
    from different starts need not agree.  A zero head gives zero
    compensators."""
    torch = torch_cuda()
    g = lib()
    nh, dk, dv, r = 6, 128, 128, 1
    gen = synth.misc_rng(31, 0)
    X = np.zeros((nh, dk, dv))
    for h in range(1, nh):
        # entries are signed powers of two (so a * v0 is exact and the GPU's
        # fused multiply-adds cancel each pair exactly too), close to a
        # rank-1 pattern so the leading singular pair is well separated
        B = 10.0 * np.outer(gen.standard_normal(dk), gen.standard_normal(dv // 2))
        A = np.sign(B) * 2.0 ** np.clip(np.round(np.log2(np.abs(B) + 1e-30)), -6, 8)
        A[:, 5] *= 4.0
        X[h, :, 0::2] = A
        X[h, :, 1::2] = -A
    X = X.astype(np.float32)
    assert np.all(X.sum(axis=2) == 0)
    cfgc = dict(B=1, H=nh, dk=dk, dv=dv, W=4, r=r, decay="scalar", io="f32")
    d = desc_for(cfgc, flags=g.DEBUG_PREQUANT)
    st = g.alloc_state(d)
    say("restart path")
    g.gdn_state_quantize(d, dev(X), st)
    torch.cuda.synchronize()
    ref = oracle.compress(X.astype(np.float64), r, 20)
    p = host(st["comp_k"]).reshape(nh, r, dk).astype(np.float64)
    w = host(st["comp_v"]).reshape(nh, r, dv).astype(np.float64)
    assert np.all(p[0] == 0) and np.all(w[0] == 0)
    C = np.einsum("hci,hcj->hij", p, w)
    Cr = np.einsum("hci,hcj->hij", ref["p"].astype(np.float64), ref["w"].astype(np.float64))
    scale = np.maximum(np.sqrt(np.sum(X.astype(np.float64) ** 2, axis=(1, 2))), 1e-30)
    err = np.sqrt(np.sum((C - Cr) ** 2, axis=(1, 2))) / scale
    assert err.max() <= 1e-4, err
