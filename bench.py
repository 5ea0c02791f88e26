"""Benchmark: INT8 per-step decode of many concurrent GDN states on one GPU.

Workload (default, "prefix_cache"): B=1024 states x H=32 heads of 128x128,
pre-filled N(0,1) with 4 outlier key rows and 4 outlier value columns per
head scaled x50, bf16 q/k/v, scalar gate.  One step = one call of
gdn_quant_decode_step over all 32768 states (dequantize, gated delta
update, output, requantize, write back).  The fp32-state kernel
(gdn_fp32_decode_step) is timed on the same states and inputs beside it.

Printed: one JSON line (metric, value = token-head updates/s, roofline of
the decode kernel against 8 TB/s HBM, and the plain fp64 CPU oracle timed
on a bounded sample of the same workload).  The line also carries, under
"window", the three window-mode workloads run as their configurations
state them over their whole length (gdn_serving, kda, damp: decode steps
and flushes, each with its own roofline and oracle baseline).

    python bench.py [--steps 100] [--warmup 200] [--gpus 1]
                    [--workload prefix_cache|gdn_serving|kda|damp|tiny|prefill|prefill_kda]
                    [--no-cpu] [--no-window] [--bits 8|6|4] [--copy-calibration]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

import synth  # noqa: E402

HBM_PEAK_GBS = 8000.0
PROFILES = os.path.join(ROOT, "profiles")


def log(*a):
    print("[bench]", *a, file=sys.stderr, flush=True)


# the sources each kernel family is compiled from (the launcher prototypes in
# launchers.hpp and the host checks in api.cpp do not change device code)
KERNEL_SOURCES = {
    "step": ("decode.hip", "tile.hpp", "codec.hpp", "launch.hpp"),
    "window": ("window.hip", "tile.hpp", "codec.hpp", "launch.hpp"),
    "prefill": ("prefill.hip", "launch.hpp"),
    "prefill_kda": ("prefill_kda.hip", "launch.hpp"),
}


def kernel_family(tag: str) -> str:
    if tag.startswith("step_"):
        return "step"
    if tag.startswith(("window_step", "flush")):
        return "window"
    if tag.startswith("prefill_kda"):
        return "prefill_kda"
    return "prefill"


def code_text(src: str) -> str:
    """A source's code without its comments and with whitespace runs
    collapsed (the kernel sources hold no comment markers inside literals)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def src_hash(family: str) -> str:
    """Hash of one kernel family's code (comments and layout aside), to tell
    whether stored counters still describe the current kernels."""
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "recurrent_state_quantization_amd", "csrc")
    for f in KERNEL_SOURCES[family]:
        with open(os.path.join(csrc, f), encoding="utf-8") as fh:
            h.update((f + "\n" + code_text(fh.read())).encode())
    return h.hexdigest()[:16]


def step_bytes(cfg: dict, quant: bool) -> int:
    """Algorithmic HBM bytes of one per-step decode of one state."""
    dk, dv = cfg["dk"], cfg["dv"]
    io = 2 if cfg["io"] == "bf16" else 4
    na = dk if cfg["decay"] == "channel" else 1
    inputs = (2 * dk + dv) * io + 4 * na + 4
    out = dv * io
    if quant:
        state = dk * dv * cfg.get("bits", 8) // 8 + 4 * (dk + dv)   # codes + row and column scales
    else:
        state = 4 * dk * dv
    return 2 * state + inputs + out             # read + write the state


def window_step_bytes(cfg: dict, t: int) -> int:
    """Algorithmic bytes of one window decode step at position t."""
    dk, dv, r = cfg["dk"], cfg["dv"], cfg["r"]
    n_hp = cfg.get("n_hp", 0)
    io = 2 if cfg["io"] == "bf16" else 4
    na = dk if cfg["decay"] == "channel" else 1
    rows = dk - n_hp
    state = rows * dv * cfg.get("bits", 8) // 8 + (0 if n_hp else 4 * dk) + 4 * dv + 2 * n_hp * dv + 4 * n_hp
    comps = 4 * r * (dk + dv)
    buf = t * 4 * (dk + dv)
    g = 4 * na * (2 if t > 0 else 1)
    inputs = (2 * dk + dv) * io + 4 * na + 4
    return state + comps + buf + g + inputs + dv * io + 4 * (dk + dv)


def flush_bytes(cfg: dict, n: int) -> int:
    dk, dv, r = cfg["dk"], cfg["dv"], cfg["r"]
    n_hp = cfg.get("n_hp", 0)
    na = dk if cfg["decay"] == "channel" else 1
    rows = dk - n_hp
    state = rows * dv * cfg.get("bits", 8) // 8 + (0 if n_hp else 4 * dk) + 4 * dv + 2 * n_hp * dv + 4 * n_hp
    comps = 4 * r * (dk + dv)
    return 2 * (state + comps) + n * 4 * (dk + dv) + 8 * na


MFMA_BF16_PEAK_TFLOPS = 2500.0   # MI355X dense bf16 matrix peak


def prefill_chunk_flops(D: int, C: int = 64) -> int:
    """Algorithmic flops of one C-token chunk (C = 64 or 32) of one head in
    the chunk form (each product of the form counted once; the second bf16
    parts that keep fp32 accuracy are not counted): K K^T and Q K^T on the
    lower 16x16 tiles (10 or 3), the triangular inverse (forward
    substitution on the 16x16 diagonal blocks, then the block merges: 16 or
    2 block products), the two C x C x D products (W and U, or U and T1 (K S)),
    the two C x D x D products (W S and Q S, or K S and Q S), the causal
    P U' (6 of 8 or 3 of 4 blocks) and the state update (D x C x D)."""
    nb = C // 16
    gram = 2 * (nb * (nb + 1) // 2) * 16 * 16 * D * 2
    merges, (pn, pd) = {64: (16, (6, 8)), 32: (2, (3, 4))}[C]
    inv = 2 * (nb * 16 * 120 + merges * 16 * 16 * 16)
    return gram + inv + 2 * (2 * C * C * D) + 2 * (2 * C * D * D) + (pn * C * C * D * 2) // pd + 2 * D * C * D


def prefill_kda_chunk_flops(D: int, C: int = 16) -> int:
    """Algorithmic flops of one C-token chunk of one head in the per-channel
    chunk form (each product counted once, second bf16 parts not counted):
    the decayed Gram sums (A on the C(C-1)/2 pairs below the diagonal, P on
    the C(C+1)/2 pairs with it, D channels each), the forward substitution,
    W and U (C x C x D each), U - W S and (Q . e^G) S (C x D x D each), P U'
    (C x C x D) and the state update (D x C x D)."""
    gram = 2 * (C * (C - 1) // 2 + C * (C + 1) // 2) * D
    inv = 2 * C * (C * (C - 1) // 2)
    return gram + inv + 2 * (2 * C * C * D) + 2 * (2 * C * D * D) + 2 * C * C * D + 2 * D * C * D


def prefill_bytes(cfg: dict, T: int) -> int:
    """Algorithmic HBM bytes of one prefill call: q, k, v read and o written
    once (bf16), a (one value per head, or dk per head for the per-channel
    gate) and b read once, each head's fp32 state read and written once."""
    B, H, D = cfg["B"], cfg["H"], cfg["dk"]
    hk = cfg.get("hk", H)
    na = D if cfg["decay"] == "channel" else 1
    per_token = B * (hk * 2 * D * 2 + H * (2 * D * 2 + 4 * na + 4))
    return T * per_token + B * H * 2 * D * D * 4


def _stored(kernel: str, workload: str):
    path = os.path.join(PROFILES, "traffic.json")
    if not os.path.exists(path):
        return {}
    with open(path) as f:
        return json.load(f).get(workload, {}).get(kernel, {})


def stored_traffic(kernel: str, workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary,
    if it was taken on the current kernel sources."""
    ent = _stored(kernel, workload)
    if not ent or ent.get("src_hash") != src_hash(kernel_family(kernel)):
        return None
    return ent["bytes_per_launch"]


def stored_valu_busy(kernel: str, workload: str):
    """VALU busy (share of SIMD cycles issuing VALU work) from the committed
    counter summary, if it was taken on the current kernel sources."""
    ent = _stored(kernel, workload)
    if not ent or ent.get("valu_src_hash") != src_hash(kernel_family(kernel)):
        return None
    return ent["valu_busy"]


def window_traffic(workload: str, W: int):
    """HBM bytes of one window (W decode steps and the flush) from the
    committed counters: the window step's mean bytes per dispatch (taken
    over whole windows, so over every position equally) times W, plus the
    flush's; None unless both were taken on the current kernel sources."""
    step, flush = stored_traffic("window_step", workload), stored_traffic("flush", workload)
    return None if step is None or flush is None else step * W + flush


def _oracle_int8_run(S: np.ndarray, inputs: list, budget_s: float, bits: int = 8):
    """Consecutive per-step quantized decodes (b-bit codes) of the states S
    by the fp64 CPU oracle (one thread) until budget_s has passed:
    (updates, steps, s)."""
    import oracle

    nh = S.shape[0]
    Q, s, c = oracle.quantize(S, bits=bits)
    done, step = 0, 0
    t0 = time.perf_counter()
    while True:
        inp = inputs[step % len(inputs)]
        r = oracle.quant_step(Q, s, c, inp["q"], inp["k"], inp["v"], inp["a"], inp["b"], bits=bits)
        Q, s, c = r["Q"], r["s"], r["c"]
        done += nh
        step += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return done, step, time.perf_counter() - t0


def _slice_inputs(inputs: list, lo: int, hi: int) -> list:
    return [{k: v[lo:hi] for k, v in inp.items()} for inp in inputs]


def _oracle_fp32_run(S: np.ndarray, inputs: list, budget_s: float):
    """Consecutive steps of the unquantized recurrence (the fp32-state
    comparator, kept in fp64 by the oracle) on the states S until budget_s
    has passed: (updates, steps, s)."""
    import oracle

    nh = S.shape[0]
    done, step = 0, 0
    t0 = time.perf_counter()
    while True:
        inp = inputs[step % len(inputs)]
        S, _ = oracle.recur(S, inp["q"][None], inp["k"][None], inp["v"][None], inp["a"][None], inp["b"][None])
        done += nh
        step += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    return done, step, time.perf_counter() - t0


# (mode, states, inputs, heads per worker, budget, bits) shared with forked workers
_CPU_JOB = None


def _cpu_worker(i: int):
    mode, S, inputs, per, budget, bits = _CPU_JOB
    sl = _slice_inputs(inputs, i * per, (i + 1) * per)
    if mode == "int8":
        return _oracle_int8_run(S[i * per:(i + 1) * per], sl, budget, bits)
    return _oracle_fp32_run(S[i * per:(i + 1) * per], sl, budget)


# One GPU's share of the host on the GPU machines: worker pools stay within
# 16 processes whatever the affinity mask shows.
HOST_SHARE = 16


def host_cores() -> dict:
    """Cores the all-core CPU legs use: the affinity mask, limited by a
    cgroup CPU quota when one is set and by the one-GPU host share."""
    aff = len(os.sched_getaffinity(0))
    quota = None
    try:
        with open("/sys/fs/cgroup/cpu.max") as f:
            q, per = f.read().split()[:2]
            if q != "max":
                quota = int(q) / int(per)
    except (OSError, ValueError):
        pass
    n = aff
    if quota is not None:
        n = min(n, max(1, int(quota)))
    n = max(1, min(n, HOST_SHARE))
    return {"used": n, "affinity": aff, "cgroup_quota": quota, "host_share": HOST_SHARE}


def _all_cores(mode, S, inputs, per, budget, bits, cores):
    global _CPU_JOB
    import multiprocessing

    _CPU_JOB = (mode, S, inputs, per, budget, bits)
    with multiprocessing.get_context("fork").Pool(cores) as pool:
        res = pool.map(_cpu_worker, range(cores))
    _CPU_JOB = None
    return sum(r[0] for r in res), max(r[2] for r in res)


def cpu_baselines(cfg: dict, S: np.ndarray, inputs: list) -> dict:
    """The fp64 CPU oracle timed on bounded samples of the workload: the
    per-step INT8 decode on one thread (the reported baseline) and on all
    usable host cores as independent processes over disjoint heads, and the
    unquantized recurrence (the fp32-state mode) the same two ways.  Runs
    before anything touches the GPU, so the workers are plain forks."""
    import oracle  # noqa: F401  (built before forking)

    total = cfg["B"] * cfg["H"]
    nh1 = 2048
    bits = cfg.get("bits", 8)
    done, step, dt = _oracle_int8_run(S[:nh1], _slice_inputs(inputs, 0, nh1), 10.0, bits)
    one = {"value": done / dt, "unit": "token-head updates/s", "cores": 1, "kind": "oracle",
           "sample": f"first {nh1} of the {total} states, {step} consecutive per-step {bits}-bit decode "
                     f"steps ({done} token-head updates) in {dt:.1f} s, one thread"}

    hc = host_cores()
    n = hc["used"]
    per = min(512, total // n)
    done_all, dt_all = _all_cores("int8", S, inputs, per, 6.0, bits, n)
    allc = {"value": done_all / dt_all, "unit": "token-head updates/s", "cores": n, "kind": "oracle",
            "host": hc,
            "sample": f"{n} processes, each on its own {per} states (the first {n * per} of {total}), "
                      f"consecutive per-step {bits}-bit decode steps for ~6 s: {done_all} token-head updates "
                      f"in {dt_all:.1f} s"}

    nh32 = 512
    done32, step32, dt32 = _oracle_fp32_run(S[:nh32], _slice_inputs(inputs, 0, nh32), 4.0)
    f32 = {"value": done32 / dt32, "unit": "token-head updates/s", "cores": 1, "kind": "oracle",
           "sample": f"first {nh32} states, {step32} consecutive steps of the unquantized recurrence "
                     f"in fp64 ({done32} token-head updates) in {dt32:.1f} s, one thread"}
    done32a, dt32a = _all_cores("fp32", S, inputs, per, 4.0, bits, n)
    f32a = {"value": done32a / dt32a, "unit": "token-head updates/s", "cores": n, "kind": "oracle",
            "host": hc,
            "sample": f"{n} processes, each on its own {per} states, consecutive steps of the unquantized "
                      f"recurrence in fp64 for ~4 s: {done32a} token-head updates in {dt32a:.1f} s"}
    return {"cpu_baseline": one, "cpu_baseline_all_cores": allc, "cpu_baseline_fp32_state": f32,
            "cpu_baseline_fp32_state_all_cores": f32a}


def settle(torch, fn, min_calls: int = 300, min_s: float = 0.3):
    """Untimed calls until at least `min_calls` have run and `min_s` of wall
    time has passed (checked every 50 calls): the GPU reaches its steady
    clocks under sustained load (the first ~200 calls after an idle spell
    run up to ~40% slower).  Reported in the JSON line; the timed region
    stays exactly --steps calls.  Returns (calls, seconds)."""
    calls = 0
    t0 = time.perf_counter()
    while True:
        for _ in range(50):
            fn(calls)
            calls += 1
        torch.cuda.synchronize()
        if calls >= min_calls and time.perf_counter() - t0 >= min_s:
            return calls, time.perf_counter() - t0


def time_launches(torch, fn, steps: int, warmup: int):
    """Run `warmup` untimed calls, then time exactly `steps` calls: the wall
    time from a synchronize before to a synchronize after, and the mean
    duration of a call from two HIP events recorded on the launch stream
    (the library launches on torch's current stream), one before the first
    timed call and one after the last, divided by `steps`.  Events between
    the calls would sit in the stream between the launches and add their
    own cost to every call, so only two more are recorded: after the first
    timed call and before the last, giving the durations of those two calls
    (a clock ramp shows as a first call slower than the last).  Returns
    (wall seconds, mean per-call seconds, first call seconds, last call
    seconds) of the same `steps` calls."""
    for i in range(warmup):
        fn(i)
    stream = torch.cuda.current_stream()
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(4)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev[0].record(stream)
    for i in range(steps):
        if i == steps - 1 and steps > 1:
            ev[2].record(stream)
        fn(warmup + i)
        if i == 0 and steps > 1:
            ev[1].record(stream)
    ev[3].record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    per = ev[0].elapsed_time(ev[3]) * 1e-3 / steps
    if steps > 1:
        first, last = ev[0].elapsed_time(ev[1]) * 1e-3, ev[2].elapsed_time(ev[3]) * 1e-3
    else:
        first = last = per
    return wall, per, first, last


def prefix_cache_data():
    """Host data of the prefix_cache workload: the pre-filled fp32 states
    and 4 input sets (calls cycle through them)."""
    cfg = synth.WORKLOADS["prefix_cache"]
    log(f"generating {cfg['B'] * cfg['H']} pre-filled states")
    S = synth.prefill_states(cfg)
    inputs = [synth.step_inputs(cfg, t) for t in range(4)]
    return cfg, S, inputs


def bench_prefix_cache(args, torch, g, cfg, S, inputs, cpu):
    nh, dk, dv = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"]
    n_sets = len(inputs)

    def up(inp):
        bits = lambda n: torch.from_numpy(inp[n + "16"].view(np.int16)).cuda().view(torch.bfloat16)
        return [bits("q"), bits("k"), bits("v"), torch.from_numpy(inp["a"]).cuda(),
                torch.from_numpy(inp["b"]).cuda()]

    dev_inputs = [up(i) for i in inputs]
    bits = cfg.get("bits", 8)
    d = g.Desc(B=cfg["B"], H=cfg["H"], dk=dk, dv=dv, io_dtype=g.IO_BF16, bits=bits,
               flags=g.STATIC_SCALES if args.static else 0)
    st = g.alloc_state(d)
    S_dev = torch.from_numpy(S).cuda()
    if args.static:
        # static scales fitted on 8 calibration steps (inputs of their own,
        # steps 1000..1007 of the seeded stream) from the pre-filled states
        log("fitting static scales on 8 calibration steps")
        cal = synth.steps_inputs(cfg, 1000, 8)
        cb = lambda n: torch.from_numpy(cal[n + "16"].view(np.int16)).cuda().view(torch.bfloat16)
        g.calibrate_static_scales(d, S_dev, cb("q"), cb("k"), cb("v"), torch.from_numpy(cal["a"]).cuda(),
                                  torch.from_numpy(cal["b"]).cuda(), 8, st)
        del cal
    g.gdn_state_quantize(d, S_dev, st)
    o = torch.empty(nh * dv, dtype=torch.bfloat16, device="cuda")
    slots = None
    if args.pool:
        # a pool of args.pool slots; the B entries sit on a seeded random subset
        if args.pool < cfg["B"]:
            raise SystemExit("--pool must be at least the batch size")
        perm = synth.misc_rng(cfg["seed"], 11).permutation(args.pool)[:cfg["B"]]
        slots = torch.from_numpy(perm.astype(np.int32)).cuda()
        pst = g.alloc_state(g.Desc(B=args.pool, H=cfg["H"], dk=dk, dv=dv, io_dtype=g.IO_BF16, bits=bits))
        for name, t in st.items():
            if t is not None:
                pst[name].view(args.pool, -1)[slots.long()] = t.view(cfg["B"], -1)
        st = pst
    torch.cuda.synchronize()

    # marshalled once: the loop passes the C structs, raw pointers and the stream
    dc, sc, sh = d.c(), g.state_struct(st), torch.cuda.current_stream().cuda_stream
    ptrs = [[t.data_ptr() for t in inp] for inp in dev_inputs]
    o_p, S_p = o.data_ptr(), S_dev.data_ptr()

    if slots is None:
        def int8_step(i):
            g.gdn_quant_decode_step(dc, sc, *ptrs[i % n_sets], o_p, 0, sh)
    else:
        sl_p = slots.data_ptr()

        def int8_step(i):
            g.gdn_quant_decode_step_pool(dc, sc, args.pool, sl_p, None, *ptrs[i % n_sets], o_p, sh)

    def fp32_step(i):
        g.gdn_fp32_decode_step(dc, S_p, *ptrs[i % n_sets], o_p, sh)

    log(f"settling the GPU clocks on the {bits}-bit per-step decode")
    settle_calls, settle_s = settle(torch, int8_step)
    log(f"timing {bits}-bit per-step decode")
    wall, per, first, last = time_launches(torch, int8_step, args.steps, args.warmup)
    log("timing fp32-state decode")
    wall32, per32, first32, last32 = time_launches(torch, fp32_step, args.steps, args.warmup)
    b8 = step_bytes(cfg, True) * nh
    b32 = step_bytes(cfg, False) * nh
    step_tag = "step_fused" + ("_static" if args.static else "") + ("" if bits == 8 else f"_b{bits}")
    value = nh * args.steps / wall
    res = {
        "metric": ("token-head state updates/s, INT8 GDN per-step decode (1 GPU)" if bits == 8 else
                   f"token-head state updates/s, {bits}-bit GDN per-step decode (1 GPU)")
                  + (", static scales" if args.static else ""),
        "value": value,
        "unit": "token-head updates/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": f"int{bits} state, fp32 math, bf16 q/k/v/o",
        "data": "synthetic (seeded pre-filled states with outlier rows/columns; no weights)",
        "config": {"workload": "prefix_cache: B=1024 states, H=32, dk=dv=128, one per-step "
                               f"{'INT8' if bits == 8 else f'{bits}-bit'} decode of every state per step, "
                               "bf16 I/O, scalar gate",
                   "global_batch": cfg["B"], "heads": cfg["H"], "dk": dk, "dv": dv, "bits": bits,
                   "pool_slots": args.pool or None,
                   "parallelism": "none (1 GPU)"},
        "roofline": {"bound": "hbm", "achieved": b8 / per / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": b8 / per / 1e9 / HBM_PEAK_GBS,
                     "traffic": stored_traffic(step_tag, "prefix_cache"),
                     # the other limit: share of SIMD cycles issuing VALU work
                     "valu_busy": stored_valu_busy(step_tag, "prefix_cache"),
                     "kernel": f"step_fused_kernel<128x128, bf16, scalar gate, {bits}-bit codes"
                               + (", static scales>" if args.static else ">"),
                     "algorithmic_bytes_per_launch": b8, "mean_launch_s": per,
                     "first_call_s": first, "last_call_s": last},
        "settle": {"calls": settle_calls, "s": settle_s,
                   "note": "untimed calls of the same decode before the warm-up, until the GPU holds its "
                           "steady clocks; the timed region is exactly `steps` calls"},
        "fp32_state": {"value": nh * args.steps / wall32, "ms_per_step": wall32 / args.steps * 1e3,
                       "achieved_GBs": b32 / per32 / 1e9, "frac": b32 / per32 / 1e9 / HBM_PEAK_GBS,
                       "algorithmic_bytes_per_launch": b32, "mean_launch_s": per32,
                       "first_call_s": first32, "last_call_s": last32,
                       "traffic": stored_traffic("step_fp32", "prefix_cache")},
        "speedup_vs_fp32_state": wall32 / wall,
    }
    res["outliers"] = host_outliers(S[:256])
    res["device_copy"] = device_copy(torch)
    res["roofline"]["frac_of_device_copy"] = res["roofline"]["achieved"] / res["device_copy"]["GBs"]
    res.update(cpu or {"cpu_baseline": None})
    return res


def prefill_data(name: str = "prefill", batch: int = 0):
    cfg = dict(synth.WORKLOADS[name], **({"B": batch} if batch else {}))
    log(f"generating {cfg['T']} tokens x {cfg['B'] * cfg['H']} heads of prefill input")
    return cfg, synth.token_major_inputs(cfg, cfg["T"])


def cpu_prefill_baseline(cfg: dict, x: dict, budget_s: float = 10.0) -> dict:
    """The oracle's sequential recurrence (fp64, one thread) on the heads of
    sequence 0, 128 tokens at a time until the time budget is spent."""
    import oracle

    D, nh, step = cfg["dk"], cfg["H"], 128
    S = np.zeros((nh, D, D), np.float32)
    done, t, t0 = 0, 0, time.perf_counter()
    while time.perf_counter() - t0 < budget_s and t < cfg["T"]:
        n = min(step, cfg["T"] - t)
        f = lambda name: np.ascontiguousarray(synth.bf16_to_f32(x[name][0, t:t + n, :nh]))
        ga = x["a"][0, t:t + n, :nh, None] if cfg["decay"] == "scalar" else x["a"][0, t:t + n, :nh]
        S, _ = oracle.recur(S, f("q16"), f("k16"), f("v16"), np.ascontiguousarray(ga), x["b"][0, t:t + n, :nh])
        t += n
        done += n * nh
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "token-head updates/s", "cores": 1, "kind": "oracle",
            "sample": f"heads 0-{nh - 1} of sequence 0, tokens 0-{t - 1} of the sequential recurrence in fp64 "
                      f"({done} token-head updates) in {dt:.1f} s, one thread"}


def bench_prefill(args, torch, g, cfg, x, cpu):
    B, H, D, T = cfg["B"], cfg["H"], cfg["dk"], cfg["T"]
    nh = B * H
    bits = lambda n: torch.from_numpy(x[n].view(np.int16)).cuda().view(torch.bfloat16)
    q, k, v = bits("q16"), bits("k16"), bits("v16")
    a, b = torch.from_numpy(x["a"]).cuda(), torch.from_numpy(x["b"]).cuda()
    S = torch.zeros((nh, D, D), dtype=torch.float32, device="cuda")
    o = torch.empty((B, T, H, D), dtype=torch.bfloat16, device="cuda")
    kda = cfg["decay"] == "channel"
    d = g.Desc(B=B, H=H, dk=D, dv=D, io_dtype=g.IO_BF16, decay=g.DECAY_CHANNEL if kda else g.DECAY_SCALAR)
    dc, sh = d.c(), torch.cuda.current_stream().cuda_stream
    p = [t.data_ptr() for t in (S, q, k, v, a, b, o)]

    def call(i):
        g.gdn_prefill(dc, *p, T, sh)

    log("timing the prefill")
    settle(torch, call, min_calls=20, min_s=0.3)
    wall, per, _, _ = time_launches(torch, call, args.steps, args.warmup)
    # dk = 128: workgroups per head as the library picks them (the most of 4,
    # 2, 1 with one workgroup per CU); their chunk-local work repeats
    ncu = torch.cuda.get_device_properties(0).multi_processor_count
    ns = 4 if nh * 4 <= ncu else 2 if nh * 2 <= ncu else 1
    if kda:
        flops = prefill_kda_chunk_flops(D) * nh * ((T + 15) // 16)
        tag, kernel = "prefill_kda", f"prefill_kda_ws_kernel<{D}, {ns}>" if D == 128 else f"prefill_kda_kernel<{D}>"
    else:
        C = 32 if D == 128 else 64
        flops = prefill_chunk_flops(D, C) * nh * ((T + C - 1) // C)
        tag, kernel = "prefill", f"prefill_ws_kernel<{D}, {ns}>" if D == 128 else f"prefill_kernel<{D}>"
    nbytes = prefill_bytes(cfg, T)
    res = {
        "metric": f"token-head state updates/s, chunkwise {'KDA' if kda else 'GDN'} prefill (1 GPU)",
        "value": nh * T * args.steps / wall, "unit": "token-head updates/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
        "dtype": "bf16 q/k/v/o, bf16 MFMA with split fp32 operands"
                 + (", fp32 MFMA for the decayed Gram sums" if kda else "") + ", fp32 state",
        "data": "synthetic (seeded; no weights)",
        "config": {"workload": f"{tag}: B={B} sequences x H={H} heads x T={T} tokens, dk=dv={D}, bf16 I/O, "
                               f"{'per-channel' if kda else 'scalar'} gate, zero initial state",
                   "B": B, "H": H, "T": T, "dk": D},
        "roofline": {"bound": "mfma", "achieved": flops / per / 1e12, "peak": MFMA_BF16_PEAK_TFLOPS,
                     "unit": "TFLOP/s", "frac": flops / per / 1e12 / MFMA_BF16_PEAK_TFLOPS,
                     "traffic": stored_traffic(tag, tag) if B == synth.WORKLOADS[tag]["B"] else None,
                     "kernel": kernel, "algorithmic_flops_per_launch": flops,
                     "mean_launch_s": per},
        "hbm": {"algorithmic_bytes_per_launch": nbytes, "achieved_GBs": nbytes / per / 1e9,
                "frac": nbytes / per / 1e9 / HBM_PEAK_GBS},
    }
    res.update({"cpu_baseline": cpu})
    return res


WINDOW_CHUNK = 256   # decode steps per graph of the full-length window runs


def cpu_window_baseline(name: str, budget_s: float = 8.0) -> dict:
    """The fp64 oracle in window mode on 4 heads of the workload (B=1, H=4,
    its distributions and seed): the window start as the workload defines
    it (512 unquantized warm-up steps for gdn_serving, zero otherwise; DAMP
    rows from the oracle's calibration over the workload's calibration
    steps), then the workload's T decode steps, window by window (decode
    and flush: compensators and the codec), until T or budget_s is reached.
    The window-start work is not timed."""
    import oracle

    cfg = dict(synth.WORKLOADS[name], B=1, H=4)
    nh, dk, dv, W, r, T = 4, cfg["dk"], cfg["dv"], cfg["W"], cfg["r"], cfg["T"]
    S = np.zeros((nh, dk, dv))
    t_start = 0
    if cfg.get("s0") == "warmup":
        w = synth.steps_inputs(cfg, 0, cfg["warmup"])
        S, _ = oracle.recur(S, w["q"], w["k"], w["v"], w["a"], w["b"])
        t_start = cfg["warmup"]
    hp = None
    if cfg.get("n_hp"):
        cal = synth.calib_inputs(cfg, cfg["n_cal"])
        hp, _ = oracle.calibrate(np.zeros((nh, dk, dv), np.float32), cal["k"], cal["v"], cal["a"], cal["b"],
                                 cfg["n_hp"])
    enc = oracle.compress(S, r, 20, hp_idx=hp)
    done, t = 0, 0
    t0 = time.perf_counter()
    while t < T and time.perf_counter() - t0 < budget_s:
        x = synth.steps_inputs(cfg, t_start + t, W)
        if hp is None:
            X0 = oracle.state_base(enc["Q"], enc["s"], enc["c"], enc["p"], enc["w"])
        else:
            X0 = oracle.state_base(enc["Q"], None, enc["c"], enc["p"], enc["w"], hp_idx=hp, hp_rows=enc["hp_rows"])
        _, _, SW = oracle.window(X0, x["q"], x["k"], x["v"], x["a"], x["b"])
        enc = oracle.compress(SW, r, 20, hp_idx=hp)
        t += W
        done += W * nh
    dt = time.perf_counter() - t0
    return {"value": done / dt, "unit": "token-head updates/s", "cores": 1, "kind": "oracle",
            "sample": f"4 heads of the {name} workload (B=1, H=4, same distributions), steps 0-{t - 1} of its "
                      f"T={T} in windows of {W} with {r} compensators"
                      + (f" and {cfg['n_hp']} fp16 rows" if hp is not None else "")
                      + f", decode and flush: {done} token-head updates in {dt:.1f} s, one thread"}


def bench_window_full(args, torch, g, name: str, cpu=None) -> dict:
    """A window workload as its configuration states it, timed over its
    whole T decode steps: the window start (gdn_serving: 512 warm-up steps
    of the fp32-state kernel from zero, then the codec with its
    compensators; kda, damp: the zero state; damp: its fp16 rows chosen by
    calibrate_scales over 256 calibration steps from zero), then T steps in
    windows of W, each window W decode steps and one flush.  Inputs are
    drawn on the GPU in chunks of WINDOW_CHUNK steps (every step distinct);
    each chunk runs as one HIP graph (its windows' decode steps and
    flushes), and the timed figure is the sum of the chunks' replays
    (event pairs on the launch stream), the drawing of inputs left out."""
    cfg = dict(synth.WORKLOADS[name])
    B, H, dk, dv, W, r, T = cfg["B"], cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"], cfg["T"]
    nh = B * H
    n_hp = cfg.get("n_hp", 0)
    kda = cfg["decay"] == "channel"
    d = g.Desc(B=B, H=H, dk=dk, dv=dv, W=W, r=r, decay=g.DECAY_CHANNEL if kda else g.DECAY_SCALAR,
               io_dtype=g.IO_BF16, layout=g.LAYOUT_DAMP if n_hp else g.LAYOUT_ROWCOL, n_hp=n_hp, power_iters=20)
    st = g.alloc_state(d)
    S = torch.zeros(nh * dk * dv, dtype=torch.float32, device="cuda")
    t_start = 0
    if cfg.get("s0") == "warmup":
        log(f"{name}: {cfg['warmup']} warm-up steps of the fp32-state kernel")
        for c0 in range(0, cfg["warmup"], WINDOW_CHUNK):
            n = min(WINDOW_CHUNK, cfg["warmup"] - c0)
            x = synth.device_steps_inputs(cfg, c0, n, torch)
            o32 = torch.empty(nh * dv, dtype=torch.bfloat16, device="cuda")
            for i in range(n):
                g.gdn_fp32_decode_step(d, S, x["q"][i], x["k"][i], x["v"][i], x["a"][i], x["b"][i], o32)
        t_start = cfg["warmup"]
    if n_hp:
        log(f"{name}: calibrating the fp16 rows over {cfg['n_cal']} steps")
        cal = synth.device_steps_inputs(cfg, 0, cfg["n_cal"], torch, purpose=synth.STREAM_CALIB)
        g.calibrate_scales(d, S, cal["k"], cal["v"], cal["a"], cal["b"], cfg["n_cal"], st["hp_idx"])
        del cal
    g.gdn_state_quantize(d, S, st)
    del S
    torch.cuda.synchronize()

    chunk = max(W, (WINDOW_CHUNK // W) * W)
    x = synth.device_steps_inputs(cfg, t_start, chunk, torch)
    o = torch.empty(nh * dv, dtype=torch.bfloat16, device="cuda")
    dc, sc, sh = d.c(), g.state_struct(st), None
    ptr = {k: v.data_ptr() for k, v in x.items()}
    es = {k: v[0].numel() * v.element_size() for k, v in x.items()}   # bytes per step

    def launch_chunk(stream):
        for i in range(chunk):
            t = i % W
            g.gdn_quant_decode_step(dc, sc, ptr["q"] + i * es["q"], ptr["k"] + i * es["k"], ptr["v"] + i * es["v"],
                                    ptr["a"] + i * es["a"], ptr["b"] + i * es["b"], o.data_ptr(), t, stream)
            if t == W - 1:
                g.gdn_quant_window_flush(dc, sc, W, stream)

    stream = torch.cuda.current_stream()
    if args.eager:   # kernel launches from the host (for counter passes)
        run = lambda: launch_chunk(stream.cuda_stream)
    else:
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            launch_chunk(torch.cuda.current_stream().cuda_stream)
        torch.cuda.synchronize()
        run = graph.replay
    log(f"{name}: {T} decode steps in chunks of {chunk}")
    total = 0.0
    for c0 in range(0, T, chunk):
        if c0 > 0:
            synth.device_steps_inputs(cfg, t_start + c0, chunk, torch, out=x)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run()
        e1.record(stream)
        torch.cuda.synchronize()
        total += e0.elapsed_time(e1) * 1e-3
    # per-kernel durations of one more window, eager, on the same state
    ev_s = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(W)]
    ev_f = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    synth.device_steps_inputs(cfg, t_start + T, chunk, torch, out=x)
    for t in range(W):
        ev_s[t][0].record(stream)
        g.gdn_quant_decode_step(d, st, x["q"][t], x["k"][t], x["v"][t], x["a"][t], x["b"][t], o, t)
        ev_s[t][1].record(stream)
    ev_f[0].record(stream)
    g.gdn_quant_window_flush(d, st, W)
    ev_f[1].record(stream)
    torch.cuda.synchronize()
    t_steps = [a.elapsed_time(b) * 1e-3 for a, b in ev_s]
    t_flush = ev_f[0].elapsed_time(ev_f[1]) * 1e-3
    wcfg = dict(cfg, bits=8)
    win_bytes = (sum(window_step_bytes(wcfg, t) for t in range(W)) + flush_bytes(wcfg, W)) * nh
    nwin = T // W
    res = {
        "metric": f"token-head state updates/s, INT8 window-mode decode ({name}, 1 GPU)",
        "value": nh * T / total, "unit": "token-head updates/s", "steps": T, "timed_s": total,
        "config": {"workload": f"{name}: B={B}, H={H}, dk=dv={dk}, T={T}, W={W}, r={r}"
                               + (f", {n_hp} fp16 rows per head (calibrate_scales, {cfg['n_cal']} steps)" if n_hp else "")
                               + (", per-key-channel gate" if kda else ", scalar gate")
                               + (f", window start after {cfg['warmup']} fp32 steps" if t_start else ", zero start"),
                   "B": B, "H": H, "W": W, "r": r, "T": T, "n_hp": n_hp, "decay": cfg["decay"]},
        "data": "synthetic, drawn on the GPU (torch generator, seeded per chunk): every decode step distinct",
        "launch": (f"eager launches, {chunk} decode steps per timed chunk" if args.eager else
                   f"one HIP graph per {chunk} decode steps ({chunk // W} windows: decode steps and flushes), "
                   "replayed once per chunk of fresh inputs; timed: the replays"),
        # the whole mode, flushes included: algorithmic bytes of a window's
        # W decode steps and its flush, times the windows, over the timed sum
        "roofline": {"bound": "hbm", "achieved": win_bytes * nwin / total / 1e9, "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": win_bytes * nwin / total / 1e9 / HBM_PEAK_GBS,
                     "traffic": window_traffic(name, W),
                     "algorithmic_bytes_per_window": win_bytes, "windows": nwin,
                     "kernel": "window_step_kernel x W + flush_kernel",
                     "valu_busy": {"window_step": stored_valu_busy("window_step", name),
                                   "flush": stored_valu_busy("flush", name)}},
        "window_step_us": [round(v * 1e6, 2) for v in t_steps],
        "flush_us": t_flush * 1e6,
        "flush_share": t_flush / (t_flush + sum(t_steps)),
    }
    res["cpu_baseline"] = cpu
    return res


def window_line(args, res: dict, name: str) -> dict:
    """The full JSON line of a window workload run on its own."""
    out = {"metric": res["metric"], "value": res["value"], "unit": res["unit"], "n_gpus": 1, "steps": res["steps"],
           "warmup": 0, "ms_per_step": res["timed_s"] / res["steps"] * 1e3, "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "int8 state (fp16 rows for DAMP), fp32 math, bf16 q/k/v/o"}
    out.update({k: v for k, v in res.items() if k not in out})
    return out


def bench_window_stagger(args, torch, g, name):
    """Continuous batching on a window workload: entry b sits at window
    position (b + i) mod W at step i, so 1/W of the entries end their window
    at every step.  Each step is one pool decode call over all entries (each
    at its own position) and one pool flush call that flushes the entries at
    position W-1 (n_tokens = W) and skips the rest (n_tokens = 0).  W steps
    are captured as one HIP graph and replayed."""
    cfg = dict(synth.WORKLOADS[name], bits=args.bits)
    B, H, dk, dv, W, r = cfg["B"], cfg["H"], cfg["dk"], cfg["dv"], cfg["W"], cfg["r"]
    nh = B * H
    if cfg.get("n_hp"):
        raise SystemExit("--stagger: use a workload without DAMP rows")
    d = g.Desc(B=B, H=H, dk=dk, dv=dv, W=W, r=r, bits=args.bits,
               decay=g.DECAY_CHANNEL if cfg["decay"] == "channel" else g.DECAY_SCALAR, io_dtype=g.IO_BF16,
               power_iters=20)
    st = g.alloc_state(d)
    S = synth.random_states(cfg["seed"], nh, dk, dv, scale=0.3)
    g.gdn_state_quantize(d, torch.from_numpy(S).cuda(), st)
    steps = max(W, (args.steps // W) * W)
    dev_in = []
    for t in range(W):
        inp = synth.step_inputs(cfg, t)
        bits = lambda n: torch.from_numpy(inp[n + "16"].view(np.int16)).cuda().view(torch.bfloat16)
        dev_in.append([bits("q"), bits("k"), bits("v"), torch.from_numpy(inp["a"]).cuda(),
                       torch.from_numpy(inp["b"]).cuda()])
    o = torch.empty(nh * dv, dtype=torch.bfloat16, device="cuda")
    slots = torch.arange(B, dtype=torch.int32, device="cuda")
    tpos = [(torch.arange(B, dtype=torch.int32, device="cuda") + i) % W for i in range(W)]
    ntok = [torch.where(tp == W - 1, W, 0).to(torch.int32) for tp in tpos]

    def step(i):
        t = i % W
        g.gdn_quant_decode_step_pool(d, st, B, slots, tpos[t], *dev_in[t], o)
        g.gdn_quant_window_flush_pool(d, st, B, slots, ntok[t])

    wall_eager = time_launches(torch, step, steps, W * max(1, args.warmup // W))[0]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(W):
            step(i)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for i in range(W):
            step(i)
    torch.cuda.synchronize()
    wall, per = time_launches(torch, lambda i: graph.replay(), steps // W, max(1, args.warmup // W))[:2]
    return {
        "metric": f"token-head state updates/s, {'INT8' if args.bits == 8 else f'{args.bits}-bit'} "
                  f"window-mode decode, staggered windows ({name}, 1 GPU)",
        "value": nh * steps / wall, "unit": "token-head updates/s", "n_gpus": 1, "steps": steps,
        "warmup": args.warmup, "ms_per_step": wall / steps * 1e3, "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": f"int{args.bits} state, fp32 math, bf16 q/k/v/o",
        "data": "synthetic",
        "config": {"workload": name, "B": B, "H": H, "W": W, "r": r, "bits": args.bits, "decay": cfg["decay"],
                   "windows": "staggered: entry b at position (b + step) mod W"},
        "launch": "pool decode + pool flush per step; W steps per HIP graph, replayed",
        "eager": {"value": nh * steps / wall_eager, "ms_per_step": wall_eager / steps * 1e3},
        "roofline": None, "cpu_baseline": None,
    }


def _max_over_median(x):
    """Per head max|x| / median|x| (x: [nh, E]); the median over heads."""
    a = x.abs()
    return float((a.amax(dim=1) / a.median(dim=1).values.clamp_min(1e-30)).median())


def host_outliers(X: np.ndarray) -> dict:
    """Diagnostic: median over heads of max|x|/median|x| of the fp32 states
    and of the same states after key-row smoothing (row i divided by the
    square root of its largest magnitude)."""
    A = np.abs(X.reshape(X.shape[0], -1)).astype(np.float64)
    r = lambda a: float(np.median(a.max(axis=1) / np.maximum(np.median(a, axis=1), 1e-30)))
    Y = np.abs(X).astype(np.float64) / np.sqrt(np.maximum(np.abs(X).max(axis=2, keepdims=True), 1e-30))
    return {"state": r(A), "after_smoothing": r(Y.reshape(X.shape[0], -1))}


def bench_tiny(args, torch, g):
    """Latency of one per-step INT8 decode call on the tiny workload (4
    heads of 64x64, fp32 I/O, zero initial state): launch-bound, so the
    wall time per call from the host is reported beside the kernel's own
    duration from HIP events."""
    cfg = synth.WORKLOADS["tiny"]
    nh, dk, dv, T = cfg["B"] * cfg["H"], cfg["dk"], cfg["dv"], cfg["T"]
    d = g.Desc(B=cfg["B"], H=cfg["H"], dk=dk, dv=dv, io_dtype=g.IO_F32, bits=args.bits)
    st = g.alloc_state(d)
    g.gdn_state_quantize(d, torch.zeros(nh * dk * dv, dtype=torch.float32, device="cuda"), st)
    dev_in = []
    for t in range(T):
        inp = synth.step_inputs(cfg, t)
        dev_in.append([torch.from_numpy(inp[n]).cuda() for n in ("q", "k", "v", "a", "b")])
    o = torch.empty(nh * dv, dtype=torch.float32, device="cuda")
    torch.cuda.synchronize()

    dc, sc, sh = d.c(), g.state_struct(st), torch.cuda.current_stream().cuda_stream
    ptrs = [[x.data_ptr() for x in inp] for inp in dev_in]
    o_p = o.data_ptr()

    def step(i):
        g.gdn_quant_decode_step(dc, sc, *ptrs[i % T], o_p, 0, sh)

    wall, per = time_launches(torch, step, args.steps, args.warmup)[:2]
    return {
        "metric": "per-step INT8 decode latency, tiny workload (1 GPU)",
        "value": wall / args.steps * 1e6, "unit": "us per call (host wall clock)", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": wall / args.steps * 1e3,
        "higher_is_better": False, "scaling": "weak", "vs_baseline": None,
        "dtype": "int8 state, fp32 math, fp32 q/k/v/o", "data": "synthetic",
        "config": {"workload": "tiny: B=1, H=4, dk=dv=64, fp32 I/O, scalar gate, zero initial state"},
        "kernel_us": per * 1e6, "roofline": None, "cpu_baseline": None,
    }


def device_copy(torch, nbytes: int = 2 << 30, reps: int = 5):
    """Context for the roofline: the best of `reps` device-to-device copies
    of nbytes (torch copy_, one read and one write per byte) in the same
    run, timed with events; reported as read+write GB/s."""
    n = nbytes // 4
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    b.copy_(a)
    best = 1e9
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        best = min(best, e0.elapsed_time(e1) * 1e-3)
    del a, b
    return {"bytes": 2 * nbytes, "best_s": best, "GBs": 2 * nbytes / best / 1e9,
            "frac_of_peak": 2 * nbytes / best / 1e9 / HBM_PEAK_GBS}


def copy_calibration(torch):
    """A plain device copy of known size, for scaling the HBM counters."""
    n = 1 << 28  # 1 GiB of fp32
    a = torch.ones(n, dtype=torch.float32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(5):
        b.copy_(a)
    torch.cuda.synchronize()
    log(f"copy calibration: 5 copies of {4 * n} bytes")


def summarize_pmc(fetch_db: str, write_db: str, copy_fetch_db: str, copy_write_db: str, workload: str,
                  out_md: str | None):
    """Per-kernel mean FETCH_SIZE / WRITE_SIZE (KiB per dispatch) from two
    rocprofv3 --pmc databases, scaled by what the same counters read for
    the 1 GiB device copy of --copy-calibration; records bytes per launch
    of the decode kernels in profiles/traffic.json with the current kernel
    source hash."""
    import collections
    import sqlite3

    def means(db, counter):
        con = sqlite3.connect(db)
        rows = con.execute("select kernel_name, value from counters_collection where counter_name = ?",
                           (counter,)).fetchall()
        agg = collections.defaultdict(list)
        for k, v in rows:
            agg[k.split("(")[0]].append(v)
        return {k: float(np.mean(v)) for k, v in agg.items()}

    copy_bytes = 4 << 28
    cf = [v for k, v in means(copy_fetch_db, "FETCH_SIZE").items() if "copyBuffer" in k][0]
    cw = [v for k, v in means(copy_write_db, "WRITE_SIZE").items() if "copyBuffer" in k][0]
    fscale, wscale = copy_bytes / (cf * 1024), copy_bytes / (cw * 1024)
    fetch, write = means(fetch_db, "FETCH_SIZE"), means(write_db, "WRITE_SIZE")
    lines = [f"copy calibration: 1 GiB device copy reads FETCH_SIZE {cf:.1f} KiB, WRITE_SIZE {cw:.1f} KiB "
             f"-> scale fetch x{fscale:.4f}, write x{wscale:.4f}", "",
             "| kernel | FETCH_SIZE KiB/dispatch | WRITE_SIZE KiB/dispatch | scaled HBM bytes/launch |",
             "|---|---|---|---|"]
    path = os.path.join(PROFILES, "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    for k in sorted(fetch):
        if k not in write:
            continue
        b = fetch[k] * 1024 * fscale + write[k] * 1024 * wscale
        lines.append(f"| {k} | {fetch[k]:.1f} | {write[k]:.1f} | {b:.4g} |")
        # template arguments after the geometry: the code width is the last
        # one of the window kernels and the next-to-last of the fused step,
        # whose last one is the static-scale flag (kernel_tag)
        tag = kernel_tag(k)
        if tag:
            data.setdefault(workload, {}).setdefault(tag, {}).update({
                "bytes_per_launch": b, "src_hash": src_hash(kernel_family(tag)), "fetch_kib": fetch[k],
                "write_kib": write[k], "fetch_scale": fscale, "write_scale": wscale})
    with open(path, "w") as f:
        json.dump(data, f, indent=1)
    text = "\n".join(lines)
    print(text)
    if out_md:
        with open(out_md, "a") as f:
            f.write(text + "\n")


def summarize_trace(db: str, last: int):
    """Per-kernel dispatch count and mean duration from a rocprofv3
    --kernel-trace database, over all dispatches and over the last `last`
    dispatches of each kernel (the bench's timed calls follow its warm-up)."""
    import collections
    import sqlite3

    con = sqlite3.connect(db)
    rows = con.execute("select name, duration from kernels order by start").fetchall()
    agg = collections.defaultdict(list)
    for name, dur in rows:
        agg[name.split("(")[0]].append(dur)
    print("| kernel | dispatches | mean ns (all) | mean ns (last %d) | min ns | max ns |" % last)
    print("|---|---|---|---|---|---|")
    for k, v in sorted(agg.items(), key=lambda kv: -sum(kv[1])):
        tail = v[-last:]
        print(f"| {k} | {len(v)} | {np.mean(v):.0f} | {np.mean(tail):.0f} | {min(v)} | {max(v)} |")


def summarize_counters(db: str):
    """Per-kernel mean of every counter in a rocprofv3 --pmc database, and
    where the counters are there: VALU instructions per wave and VALU busy,
    the share of CU cycles issuing VALU work: SQ_ACTIVE_INST_VALU (quad
    cycles summed over a CU's four SIMDs) / (256 CUs x GRBM_GUI_ACTIVE per
    XCD, the database holding the sum over the 8 XCDs)."""
    import collections
    import sqlite3

    con = sqlite3.connect(db)
    rows = con.execute("select kernel_name, counter_name, value from counters_collection").fetchall()
    agg = collections.defaultdict(lambda: collections.defaultdict(list))
    for k, cn, v in rows:
        agg[k.split("(")[0]][cn].append(v)
    names = sorted({cn for d in agg.values() for cn in d})
    mcol = "SQ_VALU_MFMA_BUSY_CYCLES" in names
    print("| kernel | dispatches | " + " | ".join(names) + " | VALU/wave | VALU busy |"
          + (" matrix busy |" if mcol else ""))
    print("|---|---|" + "---|" * (len(names) + 2 + mcol))
    found = {}
    for k, d in sorted(agg.items()):
        m = {cn: float(np.mean(v)) for cn, v in d.items()}
        per_wave = m["SQ_INSTS_VALU"] / m["SQ_WAVES"] if "SQ_INSTS_VALU" in m and m.get("SQ_WAVES") else None
        # GRBM_GUI_ACTIVE sums the 8 XCDs; SQ_ACTIVE_INST_VALU sums the 256 CUs
        # and SQ_VALU_MFMA_BUSY_CYCLES the 1024 SIMDs (matrix pipes)
        busy = (m["SQ_ACTIVE_INST_VALU"] / 256 / (m["GRBM_GUI_ACTIVE"] / 8)
                if "SQ_ACTIVE_INST_VALU" in m and m.get("GRBM_GUI_ACTIVE") else None)
        mbusy = (m["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (m["GRBM_GUI_ACTIVE"] / 8)
                 if "SQ_VALU_MFMA_BUSY_CYCLES" in m and m.get("GRBM_GUI_ACTIVE") else None)
        n = len(next(iter(d.values())))
        cells = " | ".join(f"{m[cn]:.4g}" if cn in m else "" for cn in names)
        pw = f"{per_wave:.1f}" if per_wave is not None else ""
        bz = f"{100 * busy:.1f}%" if busy is not None else ""
        mb = (f" {100 * mbusy:.1f}% |" if mbusy is not None else " |") if mcol else ""
        print(f"| {k} | {n} | {cells} | {pw} | {bz} |{mb}")
        if per_wave is not None and busy is not None:
            found[k] = (per_wave, busy)
    return found


def store_valu(db: str, workload: str):
    """--summarize-counters with --workload: also record VALU per wave and
    VALU busy of the kernels the benchmark reports in profiles/traffic.json,
    under the current kernel source hash."""
    found = summarize_counters(db)
    path = os.path.join(PROFILES, "traffic.json")
    data = json.load(open(path)) if os.path.exists(path) else {}
    for k, (pw, busy) in found.items():
        tag = kernel_tag(k)
        if tag:
            data.setdefault(workload, {}).setdefault(tag, {}).update(
                {"valu_per_wave": pw, "valu_busy": busy, "valu_src_hash": src_hash(kernel_family(tag))})
    with open(path, "w") as f:
        json.dump(data, f, indent=1)


def kernel_tag(k: str):
    """The benchmark's tag of a kernel name from a rocprofv3 database."""
    if "gdnq::prefill_kda_ws_kernel" in k:   # the two-group form of the per-channel-gate prefill
        return "prefill_kda"
    if "gdnq::prefill_ws_kernel" in k:       # the two-group form of the scalar-gate prefill
        return "prefill"
    for tag in ("step_fused", "step_fp32", "window_step", "flush", "prefill_kda", "prefill"):
        if f"gdnq::{tag}_kernel" in k:
            args = [x.strip() for x in k.rstrip(">").split(",")]
            if tag == "step_fused":
                bits, static = args[-2], args[-1] == "true"
                tag += "_static" if static else ""
            else:
                bits = args[-1]
            if tag not in ("step_fp32", "prefill", "prefill_kda") and bits in ("6", "4"):
                tag += "_b" + bits
            return tag
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    # ~200 calls (~50 ms of sustained load) bring the GPU to its steady
    # clocks; the first calls after start-up run up to ~40% slower
    ap.add_argument("--warmup", type=int, default=200)
    ap.add_argument("--workload", default="prefix_cache",
                    choices=["prefix_cache", "gdn_serving", "kda", "damp", "tiny", "prefill", "prefill_kda"])
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--batch", type=int, default=0,
                    help="prefill workloads: sequences per call in place of the workload's B")
    ap.add_argument("--bits", type=int, default=8, choices=[8, 6, 4],
                    help="code width of the quantized state (default 8)")
    ap.add_argument("--pool", type=int, default=0,
                    help="prefix_cache: keep the states in a pool of this many slots, the batch on a "
                         "seeded random subset (pool entry point)")
    ap.add_argument("--static", action="store_true",
                    help="prefix_cache: fit static scales on 8 calibration steps and time the per-step decode "
                         "under them (GDNQ_STATIC_SCALES); no CPU leg")
    ap.add_argument("--stagger", action="store_true",
                    help="window workloads: entries at staggered window positions, each step followed "
                         "by a pool flush of the entries whose window ends (pool entry points)")
    ap.add_argument("--eager", action="store_true",
                    help="window workloads: launch each chunk's kernels from the host instead of a HIP graph "
                         "(for counter passes)")
    ap.add_argument("--no-window", action="store_true",
                    help="prefix_cache: leave out the window workloads' keys (gdn_serving, kda, damp)")
    ap.add_argument("--copy-calibration", action="store_true")
    ap.add_argument("--summarize-pmc", nargs=4, metavar=("FETCH_DB", "WRITE_DB", "COPY_FETCH_DB", "COPY_WRITE_DB"),
                    help="summarize rocprofv3 --pmc databases into profiles/traffic.json (no GPU needed)")
    ap.add_argument("--md", default=None, help="append the --summarize-pmc table to this file")
    ap.add_argument("--summarize-trace", metavar="TRACE_DB",
                    help="per-kernel mean durations from a rocprofv3 --kernel-trace database (no GPU needed)")
    ap.add_argument("--summarize-counters", metavar="PMC_DB",
                    help="per-kernel counter means and VALU busy from a rocprofv3 --pmc database (no GPU needed)")
    ap.add_argument("--store", action="store_true",
                    help="with --summarize-counters: record VALU per wave and busy in profiles/traffic.json "
                         "for --workload")
    args = ap.parse_args()
    if args.summarize_trace:
        summarize_trace(args.summarize_trace, args.steps)
        return
    if args.summarize_counters:
        if args.store:
            store_valu(args.summarize_counters, args.workload)
        else:
            summarize_counters(args.summarize_counters)
        return
    if args.summarize_pmc:
        summarize_pmc(*args.summarize_pmc, args.workload, args.md)
        return
    if args.static and (args.pool or args.workload != "prefix_cache"):
        print("--static applies to the plain prefix_cache workload", file=sys.stderr)
        sys.exit(2)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only: the decode path shards over independent "
              f"(batch, head) states with no exchange, and this benchmark measures one GPU's share "
              f"(asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)
    data = cpu = None
    windows = () if args.no_window else ("gdn_serving", "kda", "damp")
    wcpu = {}
    if args.workload == "prefix_cache" and not args.copy_calibration:
        data = prefix_cache_data()
        data = (dict(data[0], bits=args.bits),) + data[1:]
        if not args.no_cpu and not args.static:
            log("timing the CPU oracle")
            cpu = cpu_baselines(*data)
            for name in windows:
                log(f"timing the CPU oracle on {name}")
                wcpu[name] = cpu_window_baseline(name)
    if args.workload in ("gdn_serving", "kda", "damp") and not args.stagger and not args.no_cpu:
        log(f"timing the CPU oracle on {args.workload}")
        wcpu[args.workload] = cpu_window_baseline(args.workload)
    if args.workload in ("prefill", "prefill_kda") and not args.copy_calibration:
        data = prefill_data(args.workload, args.batch)
        cpu = None
        if not args.no_cpu:
            log("timing the CPU oracle")
            cpu = cpu_prefill_baseline(*data)
    import torch

    import recurrent_state_quantization_amd as g

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    if args.copy_calibration:
        copy_calibration(torch)
        return
    if args.workload == "prefix_cache":
        res = bench_prefix_cache(args, torch, g, *data, cpu)
        if windows and args.bits == 8 and not args.static and not args.pool:
            res["window"] = {name: bench_window_full(args, torch, g, name, wcpu.get(name)) for name in windows}
    elif args.workload in ("prefill", "prefill_kda"):
        res = bench_prefill(args, torch, g, *data, cpu)
    elif args.workload == "tiny":
        res = bench_tiny(args, torch, g)
    elif args.stagger:
        res = bench_window_stagger(args, torch, g, args.workload)
    else:
        res = window_line(args, bench_window_full(args, torch, g, args.workload, wcpu.get(args.workload)),
                          args.workload)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
