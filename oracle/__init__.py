"""fp64 CPU oracle for quantized Gated-DeltaNet / KDA recurrent-state decode.

TEST INFRASTRUCTURE ONLY: the tests, the smoke check and the benchmark's
``cpu_baseline`` leg may import this package; the library path never does.
It shares no code with the HIP library and imports nothing from it.

This module is ctypes marshalling around ``oracle.c`` (plain C, fp64,
single-threaded, built with ``-ffp-contract=off``).  Every function below
names the part of ``oracle.c`` it calls; the arithmetic and its citations
of the pages live there.

Array conventions (numpy, C-contiguous):
  * a "head" is one (batch, head) state; states are [nh, dk, dv], row i is a
    key channel, column j a value channel;
  * per-step inputs are [n, nh, ...]; ``a`` is [.., 1] per head for scalar
    (Gated DeltaNet) decay or [.., dk] for per-channel (KDA) decay;
  * q, k, v are fp32 arrays (bf16 inputs are widened exactly before they
    are passed here).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

GCC_FLAGS = ["-O2", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11"]
# GDNQ_SANITIZE=1: AddressSanitizer and UndefinedBehaviorSanitizer build with
# the ROCm toolchain's clang (the runtime the instrumented HIP library uses;
# it must be preloaded into the process)
SAN_FLAGS = ["-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
             "-shared-libsan", "-ffp-contract=off", "-fPIC", "-shared", "-std=c11"]


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so next to it (gcc; with GDNQ_SANITIZE=1,
    clang with the address and undefined-behaviour sanitizers)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < os.path.getmtime(_SRC):
        tmp = _LIB + ".tmp"
        if os.environ.get("GDNQ_SANITIZE") == "1":
            subprocess.run(["/opt/rocm/llvm/bin/clang", *SAN_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        else:
            subprocess.run(["gcc", *GCC_FLAGS, _SRC, "-o", tmp, "-lm"], check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        _lib = ctypes.CDLL(_LIB)
    return _lib


def _p(a):
    return a.ctypes.data_as(ctypes.c_void_p) if a is not None else None


def _f32(a):
    return np.ascontiguousarray(a, dtype=np.float32)


def _f64(a):
    return np.ascontiguousarray(a, dtype=np.float64)


def _a_width(a, dk):
    w = a.shape[-1]
    assert w in (1, dk)
    return 1 if w == dk and dk != 1 else 0


# ---------------------------------------------------------------- codec (c2)
def quantize(X, bits=8):
    """Layout-0 codec of each [dk, dv] tile with b-bit codes (orc_quantize):
    returns Q (unpacked, one int8 per code, in [-(2^(b-1)-1), 2^(b-1)-1]), s, c."""
    X = _f32(X)
    nh, dk, dv = X.shape
    Q = np.empty((nh, dk, dv), np.int8)
    s = np.empty((nh, dk), np.float32)
    c = np.empty((nh, dv), np.float32)
    lib().orc_quantize(nh, dk, dv, int(bits), _p(X), _p(Q), _p(s), _p(c))
    return Q, s, c


def pack_codes(Q, bits):
    """Unpacked codes [..., dv] -> the packed byte layout [..., dv*bits/8] (orc_pack_codes)."""
    Q = np.ascontiguousarray(Q, np.int8)
    dv = Q.shape[-1]
    rows = Q.size // dv
    P = np.empty(Q.shape[:-1] + (dv * bits // 8,), np.uint8)
    lib().orc_pack_codes(rows, dv, int(bits), _p(Q), _p(P))
    return P


def unpack_codes(P, dv, bits):
    """Packed bytes [..., dv*bits/8] -> unpacked codes [..., dv] (orc_unpack_codes)."""
    P = np.ascontiguousarray(P, np.uint8)
    nb = dv * bits // 8
    assert P.shape[-1] == nb
    rows = P.size // nb
    Q = np.empty(P.shape[:-1] + (dv,), np.int8)
    lib().orc_unpack_codes(rows, dv, int(bits), _p(P), _p(Q))
    return Q


def dequantize(Q, s, c):
    """(Q*c)*s in fp32 (orc_dequantize)."""
    Q = np.ascontiguousarray(Q, np.int8)
    s, c = _f32(s), _f32(c)
    nh, dk, dv = Q.shape
    X = np.empty((nh, dk, dv), np.float32)
    lib().orc_dequantize(nh, dk, dv, _p(Q), _p(s), _p(c), _p(X))
    return X


def quantize_damp(X, hp_idx):
    """DAMP split (orc_quantize_damp): returns Qc [nh,dk-n_hp,dv], c, hp_rows (uint16 fp16 bits)."""
    X = _f32(X)
    hp_idx = np.ascontiguousarray(hp_idx, np.int32)
    nh, dk, dv = X.shape
    n_hp = hp_idx.shape[1]
    Qc = np.empty((nh, dk - n_hp, dv), np.int8)
    c = np.empty((nh, dv), np.float32)
    hp = np.empty((nh, n_hp, dv), np.uint16)
    lib().orc_quantize_damp(nh, dk, dv, n_hp, _p(hp_idx), _p(X), _p(Qc), _p(c), _p(hp))
    return Qc, c, hp


def dequantize_damp(Qc, c, hp_rows, hp_idx):
    Qc = np.ascontiguousarray(Qc, np.int8)
    c = _f32(c)
    hp_rows = np.ascontiguousarray(hp_rows, np.uint16)
    hp_idx = np.ascontiguousarray(hp_idx, np.int32)
    nh, n_hp, dv = hp_rows.shape
    dk = Qc.shape[1] + n_hp
    X = np.empty((nh, dk, dv), np.float32)
    lib().orc_dequantize_damp(nh, dk, dv, n_hp, _p(hp_idx), _p(Qc), _p(c), _p(hp_rows), _p(X))
    return X


def f32_to_f16(x):
    x = _f32(x)
    h = np.empty(x.shape, np.uint16)
    lib().orc_f32_to_f16(int(x.size), _p(x), _p(h))
    return h


def f16_to_f32(h):
    h = np.ascontiguousarray(h, np.uint16)
    x = np.empty(h.shape, np.float32)
    lib().orc_f16_to_f32(int(h.size), _p(h), _p(x))
    return x


# ---------------------------------------------------------- recurrence (c1)
def recur(S, q, k, v, a, b, want_u=False):
    """n steps of the unquantized recurrence (orc_recur).

    S: [nh,dk,dv] (copied to fp64, returned updated); q,k: [n,nh,dk];
    v: [n,nh,dv]; a: [n,nh,1|dk]; b: [n,nh].  Returns (S, o[n,nh,dv]) or
    (S, o, u) when want_u.
    """
    S = _f64(S).copy()
    nh, dk, dv = S.shape
    k, v, a, b = _f32(k), _f32(v), _f32(a), _f32(b)
    q = _f32(q) if q is not None else None
    n = k.shape[0]
    kda = _a_width(a, dk)
    o = np.empty((n, nh, dv), np.float64) if q is not None else None
    u = np.empty((n, nh, dv), np.float64) if want_u else None
    lib().orc_recur(nh, dk, dv, kda, n, _p(S), _p(q), _p(k), _p(v), _p(a), _p(b), _p(o), _p(u))
    return (S, o, u) if want_u else (S, o)


# ------------------------------------------------- per-step quantized (c3)
def quant_step(Q, s, c, q, k, v, a, b, bits=8):
    """One per-step quantized decode (orc_quant_step) on copies of Q, s, c,
    requantizing to b-bit codes (Q unpacked).

    q,k: [nh,dk], v: [nh,dv], a: [nh,1|dk], b: [nh].
    Returns dict(Q, s, c, o (fp64), S_pre (fp64 state before rounding),
    S_f32 (the fp32 tensor the codec consumed)).
    """
    Q = np.ascontiguousarray(Q, np.int8).copy()
    s, c = _f32(s).copy(), _f32(c).copy()
    nh, dk, dv = Q.shape
    q, k, v, a, b = _f32(q), _f32(k), _f32(v), _f32(a), _f32(b)
    kda = _a_width(a, dk)
    o = np.empty((nh, dv), np.float64)
    S_pre = np.empty((nh, dk, dv), np.float64)
    S_f32 = np.empty((nh, dk, dv), np.float32)
    lib().orc_quant_step(nh, dk, dv, kda, int(bits), _p(Q), _p(s), _p(c), _p(q), _p(k), _p(v), _p(a),
                         _p(b), _p(o), _p(S_pre), _p(S_f32))
    return dict(Q=Q, s=s, c=c, o=o, S_pre=S_pre, S_f32=S_f32)


# ------------------------------------------------------------ window (c4/c5)
def state_base(Q, s, c, p=None, w=None, hp_idx=None, hp_rows=None, dk=None):
    """fp64 fixed state at a window start, D(Q) + sum_c p_c w_c^T (orc_state_base)."""
    Q = np.ascontiguousarray(Q, np.int8)
    c = _f32(c)
    nh, dv = c.shape
    layout = 0 if hp_idx is None else 1
    if layout == 0:
        dk = Q.shape[1]
        n_hp = 0
        s = _f32(s)
    else:
        hp_idx = np.ascontiguousarray(hp_idx, np.int32)
        hp_rows = np.ascontiguousarray(hp_rows, np.uint16)
        n_hp = hp_idx.shape[1]
        dk = Q.shape[1] + n_hp
        s = None
    r = 0 if p is None else p.shape[1]
    p = _f32(p) if p is not None else None
    w = _f32(w) if w is not None else None
    X0 = np.empty((nh, dk, dv), np.float64)
    lib().orc_state_base(nh, dk, dv, r, layout, n_hp, _p(Q), _p(s), _p(c), _p(hp_idx),
                         _p(hp_rows), _p(p), _p(w), _p(X0))
    return X0


def window(X0, q, k, v, a, b, rebuild=True):
    """Per-window decode from the fixed fp64 state X0 (orc_window).

    Returns (o [n,nh,dv], u [n,nh,dv], S_W [nh,dk,dv] or None), all fp64.
    """
    X0 = _f64(X0)
    nh, dk, dv = X0.shape
    q, k, v, a, b = _f32(q), _f32(k), _f32(v), _f32(a), _f32(b)
    n = k.shape[0]
    kda = _a_width(a, dk)
    o = np.empty((n, nh, dv), np.float64)
    u = np.empty((n, nh, dv), np.float64)
    SW = np.empty((nh, dk, dv), np.float64) if rebuild else None
    lib().orc_window(nh, dk, dv, kda, n, _p(X0), _p(q), _p(k), _p(v), _p(a), _p(b), _p(o), _p(u),
                     _p(SW))
    return o, u, SW


def compress(SW, r, iters=20, hp_idx=None, bits=8):
    """Compensators + residual + codec of each rebuilt state (orc_compress);
    layout 0 codes have b bits (unpacked), DAMP rows' codes 8.

    Returns dict(Q, s (layout 0) | hp_rows (DAMP), c, p [nh,r,dk],
    w [nh,r,dv], R (fp32 residual handed to the codec)).
    """
    SW = _f64(SW)
    nh, dk, dv = SW.shape
    layout = 0 if hp_idx is None else 1
    n_hp = 0 if hp_idx is None else hp_idx.shape[1]
    if hp_idx is not None:
        hp_idx = np.ascontiguousarray(hp_idx, np.int32)
    Q = np.empty((nh, dk - n_hp, dv), np.int8)
    s = np.empty((nh, dk), np.float32) if layout == 0 else None
    c = np.empty((nh, dv), np.float32)
    hp = np.empty((nh, n_hp, dv), np.uint16) if layout == 1 else None
    p = np.zeros((nh, max(r, 0), dk), np.float32)
    w = np.zeros((nh, max(r, 0), dv), np.float32)
    R = np.empty((nh, dk, dv), np.float32)
    lib().orc_compress(nh, dk, dv, r, iters, layout, n_hp, int(bits if layout == 0 else 8), _p(hp_idx),
                       _p(SW), _p(Q), _p(s), _p(c), _p(hp), _p(p), _p(w), _p(R))
    return dict(Q=Q, s=s, c=c, hp_rows=hp, p=p, w=w, R=R)


# ------------------------------------------------------- calibration (c6)
def calibrate(S0, k, v, a, b, n_hp):
    """DAMP row selection (orc_calibrate): returns (hp_idx [nh,n_hp] int32, score [nh,dk] fp64)."""
    S0 = _f32(S0)
    nh, dk, dv = S0.shape
    k, v, a, b = _f32(k), _f32(v), _f32(a), _f32(b)
    n = k.shape[0]
    kda = _a_width(a, dk)
    idx = np.empty((nh, n_hp), np.int32)
    score = np.empty((nh, dk), np.float64)
    lib().orc_calibrate(nh, dk, dv, kda, n, n_hp, _p(S0), _p(k), _p(v), _p(a), _p(b), _p(idx),
                        _p(score))
    return idx, score


# ------------------------------------------------------------ static scales (f4)
def quantize_static(X, rho, iota, bits=8):
    """Codes of tiles X [nh,dk,dv] under fixed rho [nh,dk], iota [nh,dv]
    (orc_quantize_static): rint of (X rho) iota, clamped."""
    X = _f32(X)
    nh, dk, dv = X.shape
    rho, iota = _f32(rho), _f32(iota)
    Q = np.empty((nh, dk, dv), np.int8)
    lib().orc_quantize_static(nh, dk, dv, int(bits), _p(X), _p(rho), _p(iota), _p(Q))
    return Q


def fit_static(S0, q, k, v, a, b, bits=8):
    """Static-scale fit (orc_fit_static) over n calibration steps from S0.
    q, k: [n,nh,dk]; v: [n,nh,dv]; a: [n,nh,1|dk]; b: [n,nh].  Returns dict
    s, rho [nh,dk]; c, iota, choice [nh,dv]; err, cand_c, cand_iota [nh,9,dv]."""
    S0 = _f32(S0)
    nh, dk, dv = S0.shape
    q, k, v, a, b = _f32(q), _f32(k), _f32(v), _f32(a), _f32(b)
    n = k.shape[0]
    kda = _a_width(a, dk)
    out = dict(s=np.empty((nh, dk), np.float32), rho=np.empty((nh, dk), np.float32),
               c=np.empty((nh, dv), np.float32), iota=np.empty((nh, dv), np.float32),
               choice=np.empty((nh, dv), np.int32), err=np.empty((nh, 9, dv), np.float64),
               cand_c=np.empty((nh, 9, dv), np.float32), cand_iota=np.empty((nh, 9, dv), np.float32))
    lib().orc_fit_static(nh, dk, dv, kda, int(bits), n, _p(S0), _p(q), _p(k), _p(v), _p(a), _p(b),
                         _p(out["s"]), _p(out["rho"]), _p(out["c"]), _p(out["iota"]), _p(out["choice"]),
                         _p(out["err"]), _p(out["cand_c"]), _p(out["cand_iota"]))
    return out


def quant_step_static(Q, s, c, rho, iota, q, k, v, a, b, bits=8):
    """One per-step decode under static scales (orc_quant_step_static) on a
    copy of Q.  Returns dict(Q, o (fp64), S_f32)."""
    Q = np.ascontiguousarray(Q, np.int8).copy()
    nh, dk, dv = Q.shape
    s, c, rho, iota = _f32(s), _f32(c), _f32(rho), _f32(iota)
    q, k, v, a, b = _f32(q), _f32(k), _f32(v), _f32(a), _f32(b)
    kda = _a_width(a, dk)
    o = np.empty((nh, dv), np.float64)
    S_f32 = np.empty((nh, dk, dv), np.float32)
    lib().orc_quant_step_static(nh, dk, dv, kda, int(bits), _p(Q), _p(s), _p(c), _p(rho), _p(iota), _p(q), _p(k),
                                _p(v), _p(a), _p(b), _p(o), _p(S_f32))
    return dict(Q=Q, o=o, S_f32=S_f32)
