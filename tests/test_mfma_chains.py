"""The kernels that use the matrix cores, compiled for gfx950 with the
library's flags, never chain a matrix instruction onto the accumulator of
one of another shape.

Such a chain (say a 16x16x32 product whose result a 16x16x16 product reads
as its accumulator input) gets no wait states from the compiler, which
treats an exactly matching accumulator as a back-to-back chain of one
shape; with a few instructions between the two, the second product read
rows of the first one's result before they were written.  The kernels keep
one shape per accumulator chain and add the results of different shapes on
the VALU, whose reads of a product's result the compiler does wait for.
This test reads the compiler's own assembly of the sources in this
repository.
"""
import concurrent.futures
import importlib.util
import os
import re
import shutil
import subprocess
import tempfile

import pytest

_spec = importlib.util.spec_from_file_location(
    "_gdnq_build", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))),
                                "recurrent_state_quantization_amd", "_build.py"))
_build = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(_build)

SOURCES = ["prefill.hip", "prefill_kda.hip", "window.hip"]


def _regs(op):
    m = re.fullmatch(r"([va])\[(\d+):(\d+)\]", op)
    if m:
        return {(m.group(1), r) for r in range(int(m.group(2)), int(m.group(3)) + 1)}
    m = re.fullmatch(r"([va])(\d+)", op)
    return {(m.group(1), int(m.group(2)))} if m else set()


def shape_switches(asm: str):
    """(line, earlier opcode, opcode) for every matrix instruction whose
    accumulator input is exactly the result of the last matrix instruction
    that wrote those registers, of another opcode, with no write to them in
    between (straight-line reading of the listing)."""
    last = {}   # destination operand text -> opcode of the matrix instruction that wrote it
    hits = []
    for n, line in enumerate(asm.splitlines(), 1):
        line = line.strip()
        if not line or line[0] in ";." or line.endswith(":"):
            continue
        parts = line.split(None, 1)
        if len(parts) < 2:
            continue
        op, rest = parts
        ops = [o.strip() for o in rest.split(",")]
        if op.startswith("v_mfma") and len(ops) > 3 and ops[3] in last and last[ops[3]] != op:
            hits.append((n, last[ops[3]], op))
        writes = _regs(ops[0]) if op.startswith(("v_", "ds_read", "global_load", "buffer_load", "scratch_load")) else set()
        for k in [k for k in last if _regs(k) & writes]:
            del last[k]
        if op.startswith("v_mfma"):
            last[ops[0]] = op
    return hits


def test_scanner_finds_a_shape_switch():
    asm = """
        v_mfma_f32_16x16x32_bf16 v[34:37], v[54:57], v[62:65], v[34:37]
        v_cvt_pk_bf16_f32 v40, v41, s0
        v_mfma_f32_16x16x16_bf16 v[34:37], v[82:83], v[54:55], v[34:37]
        v_mfma_f32_16x16x16_bf16 v[34:37], v[82:83], v[56:57], v[34:37]
        v_mfma_f32_16x16x32_bf16 v[38:41], v[54:57], v[62:65], 0
        v_mov_b32_e32 v38, v1
        v_mfma_f32_16x16x16_bf16 v[38:41], v[82:83], v[54:55], v[38:41]
    """
    hits = shape_switches(asm)
    assert [(h[1], h[2]) for h in hits] == [("v_mfma_f32_16x16x32_bf16", "v_mfma_f32_16x16x16_bf16")]


def _asm(src, out):
    cmd = [_build.HIPCC, *_build.COMMON, "--cuda-device-only", "-S", os.path.join(_build.CSRC, src), "-o", out]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    return open(out).read()


@pytest.mark.skipif(not os.path.exists(_build.HIPCC) and shutil.which("hipcc") is None, reason="hipcc not available")
def test_no_accumulator_chain_changes_shape():
    with tempfile.TemporaryDirectory() as d:
        with concurrent.futures.ThreadPoolExecutor(len(SOURCES)) as ex:
            asm = dict(zip(SOURCES, ex.map(lambda s: _asm(s, os.path.join(d, s + ".s")), SOURCES)))
    for src, text in asm.items():
        assert "v_mfma" in text, src
        hits = shape_switches(text)
        assert not hits, f"{src}: {hits[:4]}"
