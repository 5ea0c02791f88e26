"""Window-mode decode replayed from a HIP graph (torch.cuda.CUDAGraph over
the library's launches) against the same calls made eagerly.

The library launches plain kernels on the caller's stream, with no memory
set or copy nodes, so one window (W decode steps and the flush) can be
captured once and replayed.  Every kernel is deterministic, so each replay
must reproduce the eager calls bit for bit: outputs of every step, codes,
scales, compensators, the token buffer and the gate.  The replays are
interleaved with eager work (fresh inputs copied into the captured input
buffers, the eager window on a twin state) and synchronizations, and every
replay is checked."""
import numpy as np
import pytest

import synth
from tests._gpu import desc_for, lib, say, sub_cfg, torch_cuda

pytestmark = pytest.mark.gpu

STATE_KEYS = ("codes", "row_scale", "col_scale", "comp_k", "comp_v", "buf_k", "buf_u", "buf_g", "g_cur", "hp_rows")


def _window(g, d, st, ins, outs, W):
    for t in range(W):
        g.gdn_quant_decode_step(d, st, *ins[t], outs[t], t)
    g.gdn_quant_window_flush(d, st, W)


@pytest.mark.parametrize("case", [
    ("gdn_serving", dict(B=2, H=4)),
    ("damp", dict(B=1, H=6)),
], ids=["gdn_serving", "damp"])
def test_graph_replay_matches_eager(case):
    torch = torch_cuda()
    g = lib()
    cfg = sub_cfg(synth.WORKLOADS[case[0]], **case[1])
    nh, dk, dv, W = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["W"]
    d = desc_for(cfg)
    bf = cfg["io"] == "bf16"
    odt = torch.bfloat16 if bf else torch.float32
    S0 = torch.from_numpy(synth.random_states(cfg["seed"], nh, dk, dv, scale=0.3)).cuda()
    twins = []
    for _ in range(2):
        st = g.alloc_state(d)
        if cfg.get("n_hp"):
            gr = synth.misc_rng(cfg["seed"], 5)
            hp = np.stack([np.sort(gr.choice(dk, cfg["n_hp"], replace=False)) for _ in range(nh)])
            st["hp_idx"].copy_(torch.from_numpy(hp.astype(np.int32).reshape(-1)))
        g.gdn_state_quantize(d, S0, st)
        twins.append(st)
    stA, stB = twins

    def inputs(win):
        out = []
        for t in range(W):
            inp = synth.step_inputs(cfg, win * W + t)
            if bf:
                qkv = [torch.from_numpy(inp[n + "16"].view(np.int16)).view(torch.bfloat16) for n in "qkv"]
            else:
                qkv = [torch.from_numpy(inp[n]) for n in "qkv"]
            out.append(qkv + [torch.from_numpy(inp["a"]), torch.from_numpy(inp["b"])])
        return out

    host0 = inputs(0)
    ins = [[x.cuda() for x in step] for step in host0]
    oA = [torch.empty(nh * dv, dtype=odt, device="cuda") for _ in range(W)]
    oB = [torch.empty(nh * dv, dtype=odt, device="cuda") for _ in range(W)]
    torch.cuda.synchronize()

    say("graph capture", case)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        _window(g, d, stA, ins, oA, W)          # warm-up on a side stream
        _window(g, d, stB, ins, oB, W)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        _window(g, d, stA, ins, oA, W)
    torch.cuda.synchronize()

    for rep in range(3):
        say("graph replay", case, rep)
        for step, host_step in zip(ins, inputs(rep + 1)):
            for dst, src in zip(step, host_step):
                dst.copy_(src)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        _window(g, d, stB, ins, oB, W)
        torch.cuda.synchronize()
        for t in range(W):
            assert torch.equal(oA[t].view(torch.int16) if bf else oA[t], oB[t].view(torch.int16) if bf else oB[t]), \
                (rep, t)
        for key in STATE_KEYS:
            if stA.get(key) is not None:
                assert torch.equal(stA[key], stB[key]), (rep, key)
