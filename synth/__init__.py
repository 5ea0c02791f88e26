"""Seeded synthetic inputs shared by the oracle-side and the GPU-side tests.

This module draws random numbers and nothing else: it holds none of the
method's arithmetic (no recurrence, no quantizer).  Both sides of every
parity test take their inputs from here, so they see identical values.

Generators are numpy PCG64 seeded by ``SeedSequence(seed, spawn_key=...)``
with one independent stream per (purpose, step) or (purpose, head), so any
step or any head can be regenerated on its own, in any chunking.

Per decode step the draw order is q, k, v, a, b:
  * q, k ~ N(0, 1), each head's vector L2-normalised in fp64;
  * v ~ N(0, 1);
  * a ~ U[a_lo, 1): one value per head (scalar gate) or dk values per head
    (per-key-channel gate);
  * b ~ U[0, 1).
q, k, v are then rounded to the I/O dtype (fp32 or bf16, round to nearest
even); the arrays returned are fp32 holding those exact values, plus the
raw bf16 bit patterns when the I/O dtype is bf16.

The workloads below are the shapes the method is exercised on: a tiny
per-step decode, a Gated-DeltaNet serving decode in window mode, a
per-channel-decay (KDA) decode in window mode, a prefix-cache serving step
over many independent states, a long decode with DAMP rows, and a prefill
of long sequences.
"""
from __future__ import annotations

import numpy as np

# stream purposes (first element of the spawn key)
STREAM_STEP = 1      # per-step decode inputs
STREAM_PREFILL = 2   # pre-filled states (prefix-cache workload)
STREAM_CALIB = 3     # calibration inputs (separate from decode inputs)
STREAM_STATE = 4     # random test states
STREAM_MISC = 5      # anything else a test needs

WORKLOADS = {
    # Tiny GDN decode, per-step INT8, fp32 I/O, S_0 = 0.
    "tiny": dict(B=1, H=4, dk=64, dv=64, T=256, io="f32", decay="scalar", a_lo=0.90,
                 W=1, r=0, seed=0, s0="zero"),
    # GDN serving decode, window mode W=16 with 2 compensators, S_0 from 512
    # fp32 warm-up steps.
    "gdn_serving": dict(B=64, H=32, dk=128, dv=128, T=1024, io="bf16", decay="scalar",
                        a_lo=0.90, W=16, r=2, seed=1, s0="warmup", warmup=512),
    # Per-key-channel decay (KDA), window mode W=32 with 4 compensators.
    "kda": dict(B=128, H=32, dk=128, dv=128, T=2048, io="bf16", decay="channel", a_lo=0.80,
                W=32, r=4, seed=2, s0="zero"),
    # Prefix-cache serving step: 32768 independent pre-filled states, one
    # per-step INT8 decode per state per call.
    "prefix_cache": dict(B=1024, H=32, dk=128, dv=128, T=1, calls=100, io="bf16",
                         decay="scalar", a_lo=0.90, W=1, r=0, seed=3, s0="prefill",
                         outlier_rows=4, outlier_cols=4, outlier_scale=50.0),
    # Prefill: T tokens of 8 sequences x 32 heads through the chunkwise
    # prefill from a zero state (the state then goes through the codec).
    "prefill": dict(B=8, H=32, dk=128, dv=128, T=4096, io="bf16", decay="scalar", a_lo=0.90,
                    W=1, r=0, seed=5, s0="zero"),
    # The same prefill with the per-key-channel gate of the KDA workload
    # (entries U[0.80, 1.00]).
    "prefill_kda": dict(B=8, H=32, dk=128, dv=128, T=4096, io="bf16", decay="channel", a_lo=0.80,
                        W=1, r=0, seed=6, s0="zero"),
    # Long decode with DAMP rows: 8 fp16 key rows per head from calibration
    # over 256 steps, window mode W=16 with 2 compensators, KDA decay.
    "damp": dict(B=256, H=32, dk=128, dv=128, T=8192, io="bf16", decay="channel", a_lo=0.80,
                 W=16, r=2, n_hp=8, n_cal=256, seed=4, s0="zero"),
}


def rng_for(seed: int, *key: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=tuple(key))))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest even (finite inputs)."""
    u = np.ascontiguousarray(x, np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def bf16_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, np.uint16).astype(np.uint32) << 16).view(np.float32)


def _normalize(x64: np.ndarray) -> np.ndarray:
    n = np.sqrt(np.sum(x64 * x64, axis=-1, keepdims=True))
    return x64 / n


def step_inputs(cfg: dict, t: int, heads: np.ndarray | None = None, seed: int | None = None):
    """Inputs of decode step ``t`` (0-based) for all heads of ``cfg``.

    Returns dict with q, k [nh, dk], v [nh, dv], a [nh, 1|dk], b [nh] as
    fp32 (exact I/O-dtype values) and, for bf16 I/O, q16/k16/v16 bit
    patterns.  ``heads`` selects a subset (rows of the full draw).
    """
    seed = cfg["seed"] if seed is None else seed
    nh = cfg["B"] * cfg["H"]
    dk, dv = cfg["dk"], cfg["dv"]
    g = rng_for(seed, STREAM_STEP, t)
    q = _normalize(g.standard_normal((nh, dk)))
    k = _normalize(g.standard_normal((nh, dk)))
    v = g.standard_normal((nh, dv))
    na = dk if cfg["decay"] == "channel" else 1
    a = g.uniform(cfg["a_lo"], 1.0, (nh, na))
    b = g.uniform(0.0, 1.0, nh)
    if heads is not None:
        q, k, v, a, b = q[heads], k[heads], v[heads], a[heads], b[heads]
    out = dict(a=a.astype(np.float32), b=b.astype(np.float32))
    for name, x in (("q", q), ("k", k), ("v", v)):
        x32 = x.astype(np.float32)
        if cfg["io"] == "bf16":
            h = bf16_bits(x32)
            out[name + "16"] = h
            out[name] = bf16_to_f32(h)
        else:
            out[name] = x32
    return out


def steps_inputs(cfg: dict, t0: int, n: int, heads=None, seed=None):
    """Stack ``n`` steps from ``t0``: arrays get a leading [n] axis."""
    parts = [step_inputs(cfg, t0 + t, heads, seed) for t in range(n)]
    return {key: np.stack([p[key] for p in parts]) for key in parts[0]}


def token_major_inputs(cfg: dict, T: int):
    """The draws of steps 0..T-1 (``step_inputs``) laid out token-major for
    a whole sequence: q16, k16, v16 as bf16 bit patterns [B,T,H,d], b fp32
    [B,T,H] and a fp32 [B,T,H] (scalar gate) or [B,T,H,dk] (per-channel
    gate).  Filled one step at a time, so the fp32 copies of the whole
    sequence are never held."""
    B, H, dk, dv = cfg["B"], cfg["H"], cfg["dk"], cfg["dv"]
    if cfg["io"] != "bf16":
        raise ValueError("token-major inputs are built for bf16 I/O")
    ashape = (B, T, H) if cfg["decay"] == "scalar" else (B, T, H, dk)
    out = dict(q16=np.empty((B, T, H, dk), np.uint16), k16=np.empty((B, T, H, dk), np.uint16),
               v16=np.empty((B, T, H, dv), np.uint16), a=np.empty(ashape, np.float32),
               b=np.empty((B, T, H), np.float32))
    for t in range(T):
        x = step_inputs(cfg, t)
        for name in ("q16", "k16", "v16"):
            out[name][:, t] = x[name].reshape(B, H, -1)
        out["a"][:, t] = x["a"].reshape(ashape[:1] + ashape[2:])
        out["b"][:, t] = x["b"].reshape(B, H)
    return out


def calib_inputs(cfg: dict, n: int, heads=None):
    """Calibration inputs: same distributions as decode, own stream."""
    parts = []
    for t in range(n):
        nh = cfg["B"] * cfg["H"]
        g = rng_for(cfg["seed"], STREAM_CALIB, t)
        q = _normalize(g.standard_normal((nh, cfg["dk"])))
        k = _normalize(g.standard_normal((nh, cfg["dk"])))
        v = g.standard_normal((nh, cfg["dv"]))
        na = cfg["dk"] if cfg["decay"] == "channel" else 1
        a = g.uniform(cfg["a_lo"], 1.0, (nh, na))
        b = g.uniform(0.0, 1.0, nh)
        del q
        if heads is not None:
            k, v, a, b = k[heads], v[heads], a[heads], b[heads]
        d = dict(a=a.astype(np.float32), b=b.astype(np.float32))
        for name, x in (("k", k), ("v", v)):
            x32 = x.astype(np.float32)
            if cfg["io"] == "bf16":
                h = bf16_bits(x32)
                d[name + "16"] = h
                d[name] = bf16_to_f32(h)
            else:
                d[name] = x32
        parts.append(d)
    return {key: np.stack([p[key] for p in parts]) for key in parts[0]}


def prefill_state(cfg: dict, head: int) -> np.ndarray:
    """One pre-filled [dk, dv] fp32 state: N(0,1) entries, then a few
    distinct key rows and value columns scaled up (crossings get both)."""
    dk, dv = cfg["dk"], cfg["dv"]
    g = rng_for(cfg["seed"], STREAM_PREFILL, head)
    S = g.standard_normal((dk, dv))
    rows = g.choice(dk, cfg["outlier_rows"], replace=False)
    cols = g.choice(dv, cfg["outlier_cols"], replace=False)
    S[rows, :] *= cfg["outlier_scale"]
    S[:, cols] *= cfg["outlier_scale"]
    return S.astype(np.float32)


def prefill_states(cfg: dict, heads=None) -> np.ndarray:
    nh = cfg["B"] * cfg["H"]
    heads = range(nh) if heads is None else heads
    return np.stack([prefill_state(cfg, int(h)) for h in heads])


def random_states(seed: int, nh: int, dk: int, dv: int, scale: float = 1.0, tag: int = 0):
    """Plain N(0, scale^2) fp32 states for tests."""
    g = rng_for(seed, STREAM_STATE, tag)
    return (scale * g.standard_normal((nh, dk, dv))).astype(np.float32)


def misc_rng(seed: int, tag: int = 0) -> np.random.Generator:
    return rng_for(seed, STREAM_MISC, tag)


def device_steps_inputs(cfg: dict, t0: int, n: int, torch, purpose: int = STREAM_STEP, out: dict | None = None,
                        hk: int | None = None):
    """Inputs of steps t0 .. t0+n-1 drawn on the GPU with torch's generator
    (seeded by the workload seed, the stream purpose and t0), for bulk runs
    whose inputs no oracle reads: the same distributions as step_inputs
    (q, k ~ N(0,1) normalised per head, v ~ N(0,1), a ~ U[a_lo, 1), b ~
    U[0, 1)), but other values.  q, k, v come back in the I/O dtype (bf16 or
    fp32), a, b in fp32; shapes q, k [n, B*hk, dk], v [n, B*H, dv],
    a [n, B*H, 1|dk], b [n, B*H].  With `out` (a dict of such tensors, as
    returned by an earlier call) the values are written into it."""
    nh = cfg["B"] * cfg["H"]
    nk = cfg["B"] * (hk or cfg["H"])
    dk, dv = cfg["dk"], cfg["dv"]
    na = dk if cfg["decay"] == "channel" else 1
    io = torch.bfloat16 if cfg["io"] == "bf16" else torch.float32
    g = torch.Generator(device="cuda")
    g.manual_seed(int(np.random.SeedSequence(cfg["seed"], spawn_key=(purpose, t0)).generate_state(1)[0]))
    if out is None:
        out = dict(q=torch.empty((n, nk, dk), dtype=io, device="cuda"), k=torch.empty((n, nk, dk), dtype=io, device="cuda"),
                   v=torch.empty((n, nh, dv), dtype=io, device="cuda"),
                   a=torch.empty((n, nh, na), dtype=torch.float32, device="cuda"),
                   b=torch.empty((n, nh), dtype=torch.float32, device="cuda"))
    for name in ("q", "k"):
        x = torch.randn((n, nk, dk), generator=g, device="cuda")
        out[name].copy_(x / x.norm(dim=-1, keepdim=True))
    out["v"].copy_(torch.randn((n, nh, dv), generator=g, device="cuda"))
    out["a"].copy_(torch.rand((n, nh, na), generator=g, device="cuda") * (1.0 - cfg["a_lo"]) + cfg["a_lo"])
    out["a"].clamp_(max=1.0)
    out["b"].copy_(torch.rand((n, nh), generator=g, device="cuda"))
    return out

