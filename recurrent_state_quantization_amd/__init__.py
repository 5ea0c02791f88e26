"""Python binding of libgdnq.so (quantized GDN / KDA recurrent-state decode
on MI355X).

Argument marshalling only: every entry point forwards device pointers of
torch tensors and the current HIP stream to the C ABI declared in
``include/gdnq.h``; all arithmetic runs in the library's HIP kernels.
torch provides device memory and streams.  There is no CPU fallback: if the
library is missing, importing the binding raises.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libgdnq.so")

OK, EINVAL, EUNSUPPORTED, ELAUNCH = 0, 1, 2, 3
DECAY_SCALAR, DECAY_CHANNEL = 0, 1
IO_F32, IO_BF16 = 0, 1
LAYOUT_ROWCOL, LAYOUT_DAMP = 0, 1
DEBUG_PREQUANT = 1
STATIC_SCALES = 2

STATE_FIELDS = ("codes", "row_scale", "col_scale", "comp_k", "comp_v", "buf_k", "buf_u", "buf_g", "g_cur",
                "hp_rows", "hp_idx", "prequant_out")


class GdnqError(RuntimeError):
    def __init__(self, code: int, msg: str):
        super().__init__(f"gdnq error {code}: {msg}")
        self.code = code


class _Desc(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in
                ("B", "H", "dk", "dv", "W", "r", "decay", "io_dtype", "layout", "n_hp", "power_iters")]
    _fields_ += [("flags", ctypes.c_uint32), ("bits", ctypes.c_int32), ("hk", ctypes.c_int32)]


class _State(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in STATE_FIELDS]


@dataclasses.dataclass
class Desc:
    """Mirror of gdnq_desc."""
    B: int
    H: int
    dk: int = 128
    dv: int = 128
    W: int = 1
    r: int = 0
    decay: int = DECAY_SCALAR
    io_dtype: int = IO_BF16
    layout: int = LAYOUT_ROWCOL
    n_hp: int = 0
    power_iters: int = 20
    flags: int = 0
    bits: int = 8
    hk: int = 0

    @property
    def nh(self) -> int:
        return self.B * self.H

    @property
    def per_step(self) -> bool:
        return self.W == 1 and self.r == 0

    def c(self) -> _Desc:
        return _Desc(*(getattr(self, f[0]) for f in _Desc._fields_))


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with __graft_entry__.build() "
                          "(hipcc, gfx950); there is no fallback path")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(_Desc)
    S = ctypes.POINTER(_State)
    i32 = ctypes.c_int32
    sig = {
        "gdn_quant_decode_step": [D, S, P, P, P, P, P, P, i32, P],
        "gdn_quant_window_flush": [D, S, i32, P],
        "gdn_quant_decode_step_pool": [D, S, i32, P, P, P, P, P, P, P, P, P],
        "gdn_quant_window_flush_pool": [D, S, i32, P, P, P],
        "gdn_state_quantize": [D, P, S, P],
        "gdn_state_dequantize": [D, S, P, P],
        "calibrate_scales": [D, P, P, P, P, P, i32, P, P, P],
        "gdn_fp32_decode_step": [D, P, P, P, P, P, P, P, P],
        "gdn_prefill": [D, P, P, P, P, P, P, P, i32, P],
        "calibrate_static_scales": [D, P, P, P, P, P, P, i32, S, P],
        "gdnq_state_sizes": [D, ctypes.POINTER(ctypes.c_size_t * len(STATE_FIELDS))],
    }
    for name, args in sig.items():
        if not hasattr(lib, name):
            raise ImportError(f"{LIB_PATH} does not export {name}: it predates its sources; rebuild it "
                              "with __graft_entry__.build()")
        f = getattr(lib, name)
        f.argtypes = args
        f.restype = ctypes.c_int
    lib.gdnq_last_error.argtypes = []
    lib.gdnq_last_error.restype = ctypes.c_char_p
    return lib


lib = _load()


def _check(rc: int):
    if rc != OK:
        raise GdnqError(rc, lib.gdnq_last_error().decode())


def _ptr(t):
    if t is None:
        return None
    if isinstance(t, int):
        return t
    return t.data_ptr()


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    if isinstance(stream, int):
        return stream
    return stream.cuda_stream


def state_struct(state: dict) -> _State:
    """The gdnq_state of a dict of device tensors (missing or None: 0).
    Every call below also takes the struct itself, which spares a caller
    that repeats calls on the same state the per-call marshalling."""
    return _State(*(_ptr(state.get(n)) for n in STATE_FIELDS))


def _state(state) -> _State:
    return state if isinstance(state, _State) else state_struct(state)


def _desc(desc) -> _Desc:
    """Desc or an already marshalled gdnq_desc (Desc.c())."""
    return desc if isinstance(desc, _Desc) else desc.c()


# ------------------------------------------------------------------ C ABI
def gdnq_state_sizes(desc: Desc) -> list[int]:
    out = (ctypes.c_size_t * len(STATE_FIELDS))()
    _check(lib.gdnq_state_sizes(ctypes.byref(_desc(desc)), ctypes.byref(out)))
    return list(out)


def gdn_quant_decode_step(desc, state, q, k, v, a, b, o, t_in_window=0, stream=None):
    st = _state(state)
    _check(lib.gdn_quant_decode_step(ctypes.byref(_desc(desc)), ctypes.byref(st), _ptr(q), _ptr(k), _ptr(v),
                                     _ptr(a), _ptr(b), _ptr(o), int(t_in_window), _stream(stream)))


def gdn_quant_window_flush(desc, state, n_tokens, stream=None):
    st = _state(state)
    _check(lib.gdn_quant_window_flush(ctypes.byref(_desc(desc)), ctypes.byref(st), int(n_tokens),
                                      _stream(stream)))


def gdn_quant_decode_step_pool(desc, state, n_slots, slots, t_pos, q, k, v, a, b, o, stream=None):
    st = _state(state)
    _check(lib.gdn_quant_decode_step_pool(ctypes.byref(_desc(desc)), ctypes.byref(st), int(n_slots), _ptr(slots),
                                          _ptr(t_pos), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b), _ptr(o),
                                          _stream(stream)))


def gdn_quant_window_flush_pool(desc, state, n_slots, slots, n_tokens, stream=None):
    st = _state(state)
    _check(lib.gdn_quant_window_flush_pool(ctypes.byref(_desc(desc)), ctypes.byref(st), int(n_slots), _ptr(slots),
                                           _ptr(n_tokens), _stream(stream)))


def gdn_state_quantize(desc, S, state, stream=None):
    st = _state(state)
    _check(lib.gdn_state_quantize(ctypes.byref(_desc(desc)), _ptr(S), ctypes.byref(st), _stream(stream)))


def gdn_state_dequantize(desc, state, S_out, stream=None):
    st = _state(state)
    _check(lib.gdn_state_dequantize(ctypes.byref(_desc(desc)), ctypes.byref(st), _ptr(S_out), _stream(stream)))


def calibrate_scales(desc, S0, k, v, a, b, n_steps, hp_idx_out, row_score_out=None, stream=None):
    _check(lib.calibrate_scales(ctypes.byref(_desc(desc)), _ptr(S0), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                                int(n_steps), _ptr(hp_idx_out), _ptr(row_score_out), _stream(stream)))


def gdn_fp32_decode_step(desc, S, q, k, v, a, b, o, stream=None):
    _check(lib.gdn_fp32_decode_step(ctypes.byref(_desc(desc)), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                    _ptr(b), _ptr(o), _stream(stream)))


def calibrate_static_scales(desc, S0, q, k, v, a, b, n_steps, state, stream=None):
    _check(lib.calibrate_static_scales(ctypes.byref(_desc(desc)), _ptr(S0), _ptr(q), _ptr(k), _ptr(v), _ptr(a),
                                       _ptr(b), int(n_steps), _state(state), _stream(stream)))


def gdn_prefill(desc, S, q, k, v, a, b, o, T, stream=None):
    _check(lib.gdn_prefill(ctypes.byref(_desc(desc)), _ptr(S), _ptr(q), _ptr(k), _ptr(v), _ptr(a), _ptr(b),
                           _ptr(o), int(T), _stream(stream)))


# --------------------------------------------------------------- plumbing
_DTYPES = {"codes": "int8", "hp_rows": "int16", "hp_idx": "int32", "buf_g": "int32"}


def alloc_state(desc: Desc, device="cuda"):
    """Allocate the state arrays gdnq_state_sizes asks for (torch tensors,
    zero-filled; unused fields are None)."""
    import torch

    sizes = gdnq_state_sizes(desc)
    out = {}
    for name, nbytes in zip(STATE_FIELDS, sizes):
        if nbytes == 0:
            out[name] = None
            continue
        dt = getattr(torch, _DTYPES.get(name, "float32"))
        item = torch.empty((), dtype=dt).element_size()
        out[name] = torch.zeros(nbytes // item, dtype=dt, device=device)
    return out
