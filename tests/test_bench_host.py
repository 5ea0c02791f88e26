"""Host logic of bench.py (no GPU): the tags it gives rocprofv3 kernel
names, the counter summary's VALU and matrix-pipe busy fractions, the
kernel-source hash (comments and layout aside) and the stored counters keyed
by it."""
import json
import os
import sqlite3

import pytest

import bench


@pytest.mark.parametrize("name,tag", [
    ("void gdnq::step_fused_kernel<gdnq::Geom<128, 128>, true, false, 8, false>", "step_fused"),
    ("void gdnq::step_fused_kernel<gdnq::Geom<128, 128>, true, false, 8, true>", "step_fused_static"),
    ("void gdnq::step_fused_kernel<gdnq::Geom<128, 128>, true, false, 4, false>", "step_fused_b4"),
    ("void gdnq::step_fp32_kernel<gdnq::Geom<128, 128>, true, false>", "step_fp32"),
    ("void gdnq::window_step_kernel<gdnq::Geom<128, 128>, true, true, true, 8>", "window_step"),
    ("void gdnq::flush_kernel<gdnq::Geom<128, 128>, true, true, 6>", "flush_b6"),
    ("void gdnq::prefill_ws_kernel<128, 4>", "prefill"),
    ("void gdnq::prefill_kernel<64>", "prefill"),
    ("void gdnq::prefill_kda_ws_kernel<128, 1>", "prefill_kda"),
    ("void gdnq::prefill_kda_kernel<64>", "prefill_kda"),
    ("void at::native::vectorized_elementwise_kernel<4, at::native::FillFunctor<float> >", None),
])
def test_kernel_tags(name, tag):
    assert bench.kernel_tag(name) == tag


def test_counter_summary_busy_fractions(tmp_path, capsys):
    """GRBM_GUI_ACTIVE sums the 8 XCDs' cycles, SQ_ACTIVE_INST_VALU the 256
    CUs' and SQ_VALU_MFMA_BUSY_CYCLES the 1024 SIMDs': with 1e6 cycles per
    XCD, half the CUs' cycles issuing VALU and a quarter of the SIMDs'
    cycles on the matrix pipes, the summary gives 50% and 25%; values are
    means over the dispatches."""
    db = tmp_path / "run_results.db"
    con = sqlite3.connect(db)
    con.execute("create table counters_collection (kernel_name text, counter_name text, value real)")
    k = "void gdnq::flush_kernel<gdnq::Geom<128, 128>, false, false, 8>(gdnq::FlushArgs)"
    for scale in (0.5, 1.5):  # two dispatches; the means are the scale-1 values
        rows = {"GRBM_GUI_ACTIVE": 8e6, "SQ_ACTIVE_INST_VALU": 256 * 0.5e6 * scale,
                "SQ_VALU_MFMA_BUSY_CYCLES": 1024 * 0.25e6 * scale, "SQ_INSTS_VALU": 1000.0 * 64 * scale,
                "SQ_WAVES": 64.0}
        con.executemany("insert into counters_collection values (?, ?, ?)", [(k, n, v) for n, v in rows.items()])
    con.commit()
    con.close()
    found = bench.summarize_counters(str(db))
    out = capsys.readouterr().out
    (per_wave, busy), = found.values()
    assert per_wave == pytest.approx(1000.0)
    assert busy == pytest.approx(0.5)
    row = [line for line in out.splitlines() if "flush_kernel" in line][0]
    assert row.rstrip().endswith("| 1000.0 | 50.0% | 25.0% |")


def test_code_text_drops_comments_and_layout():
    a = "int a; // one\n/* two\n   lines */  int   b;\n"
    b = "int a;\nint b; // changed comment\n"
    assert bench.code_text(a) == bench.code_text(b) == "int a; int b;"


def test_stored_counters_need_the_current_source_hash(tmp_path, monkeypatch):
    fam_hash = bench.src_hash("prefill")
    data = {"prefill": {"prefill": {"bytes_per_launch": 1.5e9, "src_hash": fam_hash,
                                    "valu_busy": 0.4, "valu_src_hash": "0" * 16}}}
    (tmp_path / "traffic.json").write_text(json.dumps(data))
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    assert bench.stored_traffic("prefill", "prefill") == 1.5e9
    assert bench.stored_valu_busy("prefill", "prefill") is None      # taken on other sources
    assert bench.stored_traffic("prefill_kda", "prefill_kda") is None  # never taken
