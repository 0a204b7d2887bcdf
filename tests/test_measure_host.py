"""Host-side measurement logic, checked on the CPU with synthetic inputs.

* the profile summariser (rocprofv3 rocpd SQLite -> the text summaries under
  profiles/): kernel names map to the library's launch names, traffic is the
  counters scaled by the 1 GiB copy calibration, MFMA busy fractions divide
  by the per-XCD GUI-active cycles;
* the benchmark's reading of those summaries: traffic is used only while the
  recorded kernel source hash matches the current source.
"""

import hashlib
import os
import sqlite3

import pytest

from sparse_mixture_experts_switch_amd import profsummary as ps

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

# <MB, NBW, waves, gather, epilogue, tiled, stream, nontemporal results, skip>: tiled weights; then row-major
UP = "_ZN3smx20ffn_gemm_bf16_kernelILi10ELi3ELi8ELb1ELi0ELb1ELb1ELb1ELb1EEEvNS_8GemmArgsIDF16bEE"
DOWN = "_ZN3smx20ffn_gemm_bf16_kernelILi10ELi3ELi8ELb0ELi2ELb1ELb1ELb0ELb1EEEvNS_8GemmArgsIDF16bEE"
UP_ROWS = "_ZN3smx20ffn_gemm_bf16_kernelILi10ELi3ELi8ELb1ELi0ELb0ELb1ELb1ELb1EEEvNS_8GemmArgsIDF16bEE"
DOWN_ROWS = "void smx::ffn_gemm_bf16_kernel<10, 3, 8, false, 2, false, true, false, true>(smx::GemmArgs<__bf16>)"
NORM = "_ZN3smx15add_norm_kernelIDF16bLi2ELb0EEEvPKDv4_jS3_PKfS5_fPS1_liNS_11CombineRowsE"
NORM_C = "void smx::add_norm_kernel<bool _Accum, int, EL, bool, E>(unsigned int __vector(4) const*)"
COPY = "__amd_rocclr_copyBuffer"


def _db(path, kernels=(), counters=()):
    db = sqlite3.connect(path)
    db.execute("create table kernels (name text, start integer, end integer)")
    db.execute("create table counters_collection (kernel_name text, dispatch_id integer, counter_name text, "
               "value real)")
    db.executemany("insert into kernels values (?, ?, ?)", kernels)
    db.executemany("insert into counters_collection values (?, ?, ?, ?)", counters)
    db.commit()
    db.close()
    return str(path)


def test_short_names():
    assert ps.short_name(UP) == "ffn_up"
    assert ps.short_name(DOWN) == "ffn_down"
    assert ps.short_name(UP_ROWS) == "ffn_up_rows"
    assert ps.short_name(DOWN_ROWS) == "ffn_down_rows"
    assert ps.short_name(NORM) == "add_norm"
    assert ps.short_name(NORM_C) == "combine_add_norm"
    assert ps.short_name("void smx::route_fused_bf16_kernel<true>(smx::FusedRouteArgs)") == "route_fused"
    assert ps.short_name("smx::assign_one_kernel(smx::AssignArgs)") == "assign"
    assert ps.short_name("void smx::wgrad_res_bf16_kernel<true, true>(smx::WgradArgs)") == "bwd_dw_out"
    assert ps.short_name("_ZN3smx21wgrad_res_bf16_kernelILb0ELb0EEEvNS_9WgradArgsE") == "bwd_dw_in"
    assert ps.short_name("something_else") == "something_else"


def test_trace_summary(tmp_path):
    # durations in ns: ffn_up 100 and 300 us, ffn_down 50 us
    db = _db(tmp_path / "t.db", kernels=[(UP, 0, 100_000), (UP, 200_000, 500_000), (DOWN, 0, 50_000)])
    text = ps.trace_summary(db, "cmd")
    rows = {line.split(" | ")[0]: line.split(" | ") for line in text.splitlines() if not line.startswith("#")}
    assert rows["ffn_up"][1:5] == ["2", "200.00", "100.00", "300.00"]
    assert rows["ffn_down"][1:5] == ["1", "50.00", "50.00", "50.00"]
    assert text.splitlines()[3].startswith("ffn_up")  # largest total time first


def test_traffic_summary_scales_by_the_copy(tmp_path):
    # the 1 GiB copy reads half its bytes in FETCH_SIZE and all of them in WRITE_SIZE
    gib_kib = (1 << 30) / 1024
    fetch = _db(tmp_path / "f.db", counters=[(COPY, 1, "FETCH_SIZE", gib_kib / 2), (UP, 2, "FETCH_SIZE", 1000.0),
                                             (UP, 3, "FETCH_SIZE", 3000.0)])
    write = _db(tmp_path / "w.db", counters=[(COPY, 1, "WRITE_SIZE", gib_kib), (UP, 2, "WRITE_SIZE", 10.0),
                                             (UP, 3, "WRITE_SIZE", 30.0)])
    src = tmp_path / "k.hip"
    src.write_text("kernel source")
    text = ps.traffic_summary(fetch, write, "ffn_up", "rocprofv3 --pmc COUNTER", str(src))
    vals = dict(line.split(" = ") for line in text.splitlines() if " = " in line and not line.startswith("#"))
    assert float(vals["fetch_factor"]) == pytest.approx(2.0)
    assert float(vals["write_factor"]) == pytest.approx(1.0)
    # mean fetch 2000 KiB x 2 + mean write 20 KiB x 1
    assert float(vals["hbm_bytes_per_launch"]) == pytest.approx(2000 * 1024 * 2 + 20 * 1024)
    assert vals["source_sha256"] == hashlib.sha256(b"kernel source").hexdigest()[:16]
    assert "FETCH_SIZE pass): rocprofv3 --pmc FETCH_SIZE" in text
    with pytest.raises(SystemExit):  # no copy dispatch in the run: no calibration, no summary
        ps.traffic_summary(_db(tmp_path / "f2.db"), write, "ffn_up", "c", str(src))


def test_mfma_summary(tmp_path):
    # 8 XCDs x 1024 SIMDs; GUI active summed over XCDs = 8000 -> 1000 cycles each;
    # busy cycles summed over SIMDs = 256000 -> 25% of 1024 SIMDs x 1000 cycles
    db = _db(tmp_path / "m.db", counters=[(UP, 1, "SQ_VALU_MFMA_BUSY_CYCLES", 256000.0),
                                          (UP, 1, "GRBM_GUI_ACTIVE", 8000.0),
                                          (UP, 1, "SQ_INSTS_VALU_MFMA_MOPS_BF16", 2e9)])
    src = tmp_path / "k.hip"
    src.write_text("x")
    text = ps.mfma_summary(db, "cmd", 1024, 8, str(src))
    row = [line for line in text.splitlines() if line.startswith("ffn_up")][0].split(" | ")
    assert float(row[2]) == pytest.approx(0.25)
    assert float(row[3]) == pytest.approx(2e9 * 512 / 1e9)


def test_bench_reads_traffic_only_for_the_current_source(tmp_path, monkeypatch):
    import importlib.util
    spec = importlib.util.spec_from_file_location("bench_mod", os.path.join(ROOT, "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path))
    (tmp_path / "ffn_up_base_counters.txt").write_text(
        "# comment\nkernel = ffn_up\nsource_sha256 = abc\nhbm_bytes_per_launch = 12345\n")
    assert bench.read_traffic("ffn_up", "abc") == 12345.0
    assert bench.read_traffic("ffn_up", "def") is None      # kernel source changed since the counters
    assert bench.read_traffic("ffn_down", "abc") is None    # no summary for that kernel
