"""Host logic of the rocprofv3 summaries (no GPU): counter scaling by the
calibration copy, the markdown/JSON round trip, and staleness by the hash of
the named sources."""
import csv
import os

import pytest

from sample_grad_norms_amd import profiling


def write_csv(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def fake_runs(tmp_path, copy_kib_fetch, copy_kib_write):
    trace = tmp_path / "trace"
    write_csv(str(trace / "box" / "run_kernel_stats.csv"), ["Name", "Calls", "AverageNs", "TotalDurationNs", "Percentage"],
              [["void dpn::k_rowproj_bf16<2, 1>(dpn::StageArgs)", 4, 2000000, 8000000, 60.0],
               ["void dpn::k_tcontract_bf16<2, true>(dpn::StageArgs)", 4, 1500000, 6000000, 40.0]])
    rows_f, rows_w = [], []
    for name, f_kib, w_kib in (("__amd_rocclr_copyBuffer", copy_kib_fetch, copy_kib_write),
                               ("void dpn::k_rowproj_bf16<2, 1>(dpn::StageArgs)", 1000.0, 10.0),
                               ("void dpn::k_rowproj_bf16<2, 1>(dpn::StageArgs)", 3000.0, 30.0)):
        rows_f.append([name, "FETCH_SIZE", f_kib])
        rows_w.append([name, "WRITE_SIZE", w_kib])
    write_csv(str(tmp_path / "fetch" / "box" / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"], rows_f)
    write_csv(str(tmp_path / "write" / "box" / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"], rows_w)
    return str(trace), str(tmp_path / "fetch"), str(tmp_path / "write")


def test_scaling_by_the_copy_and_round_trip(tmp_path):
    # the copy reads 1 GiB: a FETCH_SIZE of 2^19 KiB means the counter reads half the bytes moved
    trace, fetch, write = fake_runs(tmp_path, copy_kib_fetch=float(1 << 19), copy_kib_write=float(1 << 20))
    out = str(tmp_path / "summary.md")
    block = profiling.summarize(trace, fetch, write, out, ["cmd one"], "title", sources=["kernels_hutch.hip"])
    assert block["fetch_scale"] == pytest.approx(2.0)
    assert block["write_scale"] == pytest.approx(1.0)
    rd = block["fetch_bytes_per_dispatch"]["k_rowproj_bf16<2, 1>"]
    wr = block["write_bytes_per_dispatch"]["k_rowproj_bf16<2, 1>"]
    assert rd == pytest.approx(2000.0 * 1024 * 2.0)       # mean of 1000 and 3000 KiB, times 2
    assert wr == pytest.approx(20.0 * 1024)
    assert profiling.read_traffic(out, "k_rowproj") == pytest.approx(rd + wr)
    assert profiling.read_traffic(out, "k_nothing") is None
    text = open(out).read()
    assert text.startswith("# title") and "cmd one" in text


def test_staleness_follows_only_the_named_sources(tmp_path, monkeypatch):
    trace, fetch, write = fake_runs(tmp_path, float(1 << 20), float(1 << 20))
    csrc = tmp_path / "pkg" / "csrc"
    csrc.mkdir(parents=True)
    (csrc / "a.hip").write_text("kernel a v1")
    (csrc / "b.hip").write_text("kernel b v1")
    monkeypatch.setattr(profiling, "HERE", str(tmp_path / "pkg"))
    out = str(tmp_path / "s.md")
    profiling.summarize(trace, fetch, write, out, [], "t", sources=["a.hip"])
    assert profiling.read_traffic(out, "k_rowproj") is not None
    (csrc / "b.hip").write_text("kernel b v2")            # another kernel's source: still valid
    assert profiling.read_traffic(out, "k_rowproj") is not None
    (csrc / "a.hip").write_text("kernel a v1  // a comment\n/* and\n another */")   # comments only: still valid
    assert profiling.read_traffic(out, "k_rowproj") is not None
    (csrc / "a.hip").write_text("kernel a v2")            # the profiled kernel changed: stale
    assert profiling.read_traffic(out, "k_rowproj") is None
    # without a source list the hash covers every csrc file
    out_all = str(tmp_path / "all.md")
    profiling.summarize(trace, fetch, write, out_all, [], "t")
    assert profiling.read_traffic(out_all, "k_rowproj") is not None
    (csrc / "b.hip").write_text("kernel b v3")
    assert profiling.read_traffic(out_all, "k_rowproj") is None


def test_code_text_drops_comments_and_layout():
    src = "int a; // one\n/* two\n lines */ int  b;\n\tint c;"
    assert profiling.code_text(src) == "int a; int b; int c;"
    assert profiling.code_text('asm("s_nop 0\\n\\tx");') == 'asm("s_nop 0\\n\\tx");'


def test_missing_calibration_copy_is_an_error(tmp_path):
    trace, fetch, write = fake_runs(tmp_path, 0.0, 0.0)
    with pytest.raises(ValueError):
        profiling.summarize(trace, fetch, write, str(tmp_path / "x.md"), [], "t")


def test_utilisation_summary(tmp_path):
    run = tmp_path / "pmc" / "box"
    run.mkdir(parents=True)
    rows = []
    for v in (1.0, 3.0):   # two dispatches: means 2x the base values
        rows += [["void dpn::k_rowproj_bf16<2, 1, 4>(dpn::StageArgs)", "GRBM_GUI_ACTIVE", 8e6 * v],
                 ["void dpn::k_rowproj_bf16<2, 1, 4>(dpn::StageArgs)", "SQ_VALU_MFMA_BUSY_CYCLES", 0.25e6 * 1024 * v],
                 ["void dpn::k_rowproj_bf16<2, 1, 4>(dpn::StageArgs)", "SQ_LDS_IDX_ACTIVE", 0.5e6 * 256 * v],
                 ["void dpn::k_rowproj_bf16<2, 1, 4>(dpn::StageArgs)", "SQ_LDS_BANK_CONFLICT", 0.1e6 * 256 * v],
                 ["void dpn::k_rowproj_bf16<2, 1, 4>(dpn::StageArgs)", "TCC_HIT_sum", 3.0 * v],
                 ["void dpn::k_rowproj_bf16<2, 1, 4>(dpn::StageArgs)", "TCC_MISS_sum", 1.0 * v],
                 ["__amd_rocclr_copyBuffer", "GRBM_GUI_ACTIVE", 5.0]]
    write_csv(str(run / "run_counter_collection.csv"), ["Kernel_Name", "Counter_Name", "Counter_Value"], rows)
    out = str(tmp_path / "u.md")
    means = profiling.counters_summary([str(tmp_path / "pmc")], out, ["cmd"], "title")
    assert list(means) == ["k_rowproj_bf16<2, 1, 4>"]          # library kernels only
    d = profiling.derived(means["k_rowproj_bf16<2, 1, 4>"])
    assert d["MFMA pipe busy (per SIMD)"] == pytest.approx(0.25)   # 2e6 cycles per XCD, a quarter busy
    assert d["LDS busy (indexed ops, per CU)"] == pytest.approx(0.5)
    assert d["LDS cycles stalled by bank conflicts / LDS busy"] == pytest.approx(0.2)
    assert d["L2 hit rate"] == pytest.approx(0.75)
    assert d["wave time waiting on a dependency (s_waitcnt)"] is None
    text = open(out).read()
    assert "25.0 %" in text and "75.0 %" in text
