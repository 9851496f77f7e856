"""The rocprofv3 CSV reduction behind profiles/, on small synthetic CSVs with known answers.

trace groups dispatches by (kernel, workgroups, threads) and reports their duration statistics;
traffic scales FETCH_SIZE by the streaming read of a known size in the same pass (its median or
its largest dispatch) and WRITE_SIZE by the device copy, then adds them per dispatch.
"""

import contextlib
import csv
import io

from gguf_block_quantized_qmv_amd import rocprof_summary as rs

TRACE_COLS = ["Kind", "Dispatch_Id", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "Workgroup_Size_X",
              "Workgroup_Size_Y", "Workgroup_Size_Z", "Grid_Size_X", "Grid_Size_Y", "Grid_Size_Z"]
PMC_COLS = ["Dispatch_Id", "Grid_Size", "Kernel_Name", "Workgroup_Size", "Counter_Name", "Counter_Value"]
GEMV = "void qmv::(anonymous namespace)::q4k_gemv_kernel<1, 16, 5, false, 5>(unsigned char const*, float*, int, int)"


def _write(path, cols, rows):
    path.parent.mkdir(parents=True, exist_ok=True)
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(cols)
        w.writerows(rows)


def _out(fn, argv):
    buf = io.StringIO()
    with contextlib.redirect_stdout(buf):
        fn(argv)
    return buf.getvalue()


def test_short_name_keeps_template_arguments_only():
    assert rs.short_name(GEMV) == "q4k_gemv_kernel<1, 16, 5, false, 5>"


def test_trace_groups_and_statistics(tmp_path):
    rows = []
    for i, d in enumerate([100, 300, 200, 1000]):
        rows.append(["KERNEL_DISPATCH", i + 1, GEMV, 10_000 * i, 10_000 * i + d, 256, 1, 1, 256 * 1088, 1, 1])
    rows.append(["KERNEL_DISPATCH", 9, "void other_kernel(int)", 0, 50, 64, 1, 1, 64, 1, 1])
    _write(tmp_path / "t" / "x_kernel_trace.csv", TRACE_COLS, rows)
    out = _out(rs.main, ["trace", str(tmp_path / "t"), "--kernel", "q4k_gemv", "--per-step", "2"])
    assert "| q4k_gemv_kernel<1, 16, 5, false, 5> | 1088 | 256 | 4 | 400 | 250 | 100 | 1000 |" in out
    assert "other_kernel" not in out
    assert "0.0005 ms at the group medians, 0.0008 ms at the group means" in out
    out = _out(rs.main, ["trace", str(tmp_path / "t"), "--kernel", "q4k_gemv", "--window", "1:3"])
    assert "| 2 | 250 | 250 | 200 | 300 |" in out


def test_traffic_scaling_and_read_pick(tmp_path):
    fetch = [[1, 4096, "stream_read_kernel(uint4 const*, unsigned long)", 256, "FETCH_SIZE", 1048576.0],
             [2, 4096, "stream_read_kernel(uint4 const*, unsigned long)", 256, "FETCH_SIZE", 2097152.0],
             [3, 4096, "stream_read_kernel(uint4 const*, unsigned long)", 256, "FETCH_SIZE", 1572864.0],
             [4, 256 * 1088, GEMV, 256, "FETCH_SIZE", 1000.0],
             [5, 256 * 1088, GEMV, 256, "FETCH_SIZE", 1200.0]]
    write = [[1, 4096, "__amd_rocclr_copyBuffer(char*, char*)", 256, "WRITE_SIZE", 4194304.0],
             [4, 256 * 1088, GEMV, 256, "WRITE_SIZE", 10.0],
             [5, 256 * 1088, GEMV, 256, "WRITE_SIZE", 30.0]]
    _write(tmp_path / "f" / "a_counter_collection.csv", PMC_COLS, fetch)
    _write(tmp_path / "w" / "a_counter_collection.csv", PMC_COLS, write)
    base = ["traffic", str(tmp_path / "f"), str(tmp_path / "w"), "--kernel", "q4k_gemv",
            "--read-bytes", str(float(1 << 32))]
    # max: 4 GiB read as 2 GiB of FETCH_SIZE KiB -> x 2; the copy's WRITE_SIZE is exact -> x 1
    out = _out(rs.main, base + ["--read-pick", "max", "--algo-bytes", "2273280"])
    hbm = 1100 * 1024 * 2 + 20 * 1024
    assert f"| 1088 x 256 | 2 | 1100.0 | 20.0 | {hbm} | {hbm / 2273280:.4f} |" in out
    # median: 1.5 GiB of KiB for 4 GiB -> x 8/3
    out = _out(rs.main, base)
    assert f"| {round(1100 * 1024 * 8 / 3 + 20 * 1024)} | - |" in out
