"""Host logic of the kernel-summary tool (CPU): the source stamp ignores
comments and blank space but not code, the counter summary scales each
counter by the copy calibration and reports per-launch bytes, the per-shape
percentiles come from the kernel trace, and a traffic file reads back."""
import csv
import os

import pytest

from gqa_kv_cache_decode_amd import rocprof_summary as rs


def test_code_only_ignores_comments_and_spacing():
    a = "int f(int x) {  // one\n  return x + 1; /* two\n lines */\n}\n"
    b = "int f(int x) {\n\n   return x + 1;\n}"
    c = "int f(int x) { return x + 2; }"
    assert rs._code_only(a) == rs._code_only(b)
    assert rs._code_only(a) != rs._code_only(c)


def test_source_stamp_is_stable_and_covers_the_decode_sources():
    h = rs.kernel_source_hash()
    assert len(h) == 16 and h == rs.kernel_source_hash()
    for name in rs.DECODE_SOURCES:
        assert os.path.exists(os.path.join(rs.PKG, "csrc", name)), name


def _write(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f, quoting=csv.QUOTE_NONNUMERIC)
        w.writerow(header)
        w.writerows(rows)


def test_traffic_summary_scales_by_the_copy(tmp_path):
    head = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    # a 1 GiB copy reads as 512 Ki KiB on FETCH_SIZE (half) and 1 Mi KiB on WRITE_SIZE
    _write(tmp_path / "f.csv", head, [[1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 524288.0],
                                      [2, "void decode_matrix_kernel<1>", "FETCH_SIZE", 1000.0],
                                      [3, "void decode_matrix_kernel<1>", "FETCH_SIZE", 1002.0]])
    _write(tmp_path / "w.csv", head, [[1, "__amd_rocclr_copyBuffer", "WRITE_SIZE", 1048576.0],
                                      [2, "void decode_matrix_kernel<1>", "WRITE_SIZE", 10.0]])
    text = rs.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"), "decode_matrix_kernel", 1 << 30,
                              2.0e6, "rocprofv3 --pmc PMC -- x", "wl")
    out = tmp_path / "t.txt"
    out.write_text(text)
    rec = rs.read_traffic(str(out))
    assert float(rec["fetch_scale"]) == pytest.approx(2.0) and float(rec["write_scale"]) == pytest.approx(1.0)
    assert int(rec["hbm_read_bytes_per_launch"]) == 1001 * 1024 * 2
    assert int(rec["hbm_write_bytes_per_launch"]) == 10 * 1024
    assert float(rec["traffic_over_algorithmic"]) == pytest.approx((1001 * 2048 + 10240) / 2.0e6, rel=1e-4)
    assert rec["kernel_source_hash"] == rs.kernel_source_hash()
    assert "--pmc FETCH_SIZE" in text and "--pmc WRITE_SIZE" in text


def test_traffic_summary_needs_the_kernel(tmp_path):
    head = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    _write(tmp_path / "f.csv", head, [[1, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 1.0]])
    with pytest.raises(SystemExit):
        rs.traffic_summary(str(tmp_path / "f.csv"), str(tmp_path / "f.csv"), "decode_matrix_kernel", 1 << 30, 1.0,
                           "c", "wl")


def test_stats_and_per_shape_percentiles(tmp_path):
    _write(tmp_path / "s.csv", ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
           [["k1", 3, 6000, 2000.0, 90.0, 1000, 3000]])
    text = rs.stats_summary(str(tmp_path / "s.csv"), "cmd")
    assert "# command: cmd" in text and "2.000" in text and text.rstrip().endswith("k1")
    rows = [["k1", 0, d, 256, 256 * 64] for d in (1000, 2000, 3000)] + [["k1", 0, 5000, 256, 256 * 8]]
    _write(tmp_path / "t.csv", ["Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X", "Grid_Size_X"],
           rows)
    shapes = rs.by_grid_summary(str(tmp_path / "t.csv"))
    lines = [l for l in shapes.splitlines() if l.strip().endswith("k1")]
    assert len(lines) == 2  # two launch shapes: 64 and 8 workgroups
    three = [l for l in lines if l.split()[0] == "3"][0].split()
    assert float(three[1]) == pytest.approx(2.0) and int(three[7]) == 64
