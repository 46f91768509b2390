"""Host-side logic of bench.py that turns rocprofv3 output into the committed
profile summaries, on small hand-made counter files: each summary must take
the workload kernel's dispatches only (a profiled run also holds copy, fill
and, on the s8s8 shape, vendor-library kernels), and the derived figures
must follow their definitions.  Also: the benchmark's helper libraries
export what bench.py calls."""
import csv
import ctypes
import os
import re
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

RING = "void qg::(anonymous namespace)::k_gemm_dma<8, 0, true, 4>(qg::(anonymous namespace)::DmaArgs)"
VENDOR = "Cijk_Alik_Bljk_I8II_BH_UserArgs_MT256x256x128_MI16x16x1_SN"
COPY = "__amd_rocclr_copyBuffer"
FILL = "__amd_rocclr_fillBufferAligned"
FIELDS = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp",
          "End_Timestamp"]


def _write(path, rows):
    path.mkdir(parents=True, exist_ok=True)
    with open(path / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=FIELDS)
        w.writeheader()
        for i, (kernel, counter, value, start, end) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter,
                        "Counter_Value": value, "Start_Timestamp": start, "End_Timestamp": end})


def test_traffic_takes_the_workload_kernel_only(tmp_path):
    gib_kib = (1 << 30) / 1024.0
    # FETCH_SIZE reads half of a copy's bytes, WRITE_SIZE all of them
    fetch = [(RING, "FETCH_SIZE", 400_000.0, 0, 1), (RING, "FETCH_SIZE", 410_000.0, 2, 3),
             (VENDOR, "FETCH_SIZE", 9e9, 4, 5), (FILL, "FETCH_SIZE", 0.0, 6, 7),
             (COPY, "FETCH_SIZE", gib_kib / 2, 8, 9)]
    write = [(RING, "WRITE_SIZE", 65_536.0, 0, 1), (RING, "WRITE_SIZE", 65_536.0, 2, 3),
             (VENDOR, "WRITE_SIZE", 9e9, 4, 5), (COPY, "WRITE_SIZE", gib_kib, 8, 9)]
    _write(tmp_path / "f", fetch)
    _write(tmp_path / "w", write)
    line = bench.summarize_pmc("s8s8", str(tmp_path / "f"), str(tmp_path / "w"))
    got = dict(kv.split("=") for kv in line.split()[1:])
    assert got["workload"] == "s8s8"
    assert float(got["calib_fetch"]) == pytest.approx(2.0)
    assert float(got["calib_write"]) == pytest.approx(1.0)
    assert int(got["fetch_bytes_raw"]) == 405_000 * 1024
    assert int(got["write_bytes_raw"]) == 65_536 * 1024
    assert int(got["bytes_per_launch"]) == pytest.approx(2 * 405_000 * 1024 + 65_536 * 1024, rel=1e-9)


def test_counters_clock_and_matrix_busy(tmp_path):
    # 2 dispatches of 500 us; GRBM_GUI_ACTIVE summed over 8 XCDs = 8 x 1,000,000
    # cycles -> 2000 MHz; SQ_VALU_MFMA_BUSY_CYCLES summed over 1024 SIMDs
    rows = []
    for d in range(2):
        t0 = d * 10_000_000
        rows += [(RING, "GRBM_GUI_ACTIVE", 8_000_000.0, t0, t0 + 500_000),
                 (RING, "SQ_VALU_MFMA_BUSY_CYCLES", 1024 * 600_000.0, t0, t0 + 500_000),
                 (VENDOR, "GRBM_GUI_ACTIVE", 1.0, t0, t0 + 1),
                 (VENDOR, "SQ_VALU_MFMA_BUSY_CYCLES", 5.0, t0, t0 + 1)]
    _write(tmp_path / "c", rows)
    line = bench.summarize_counters("s8s8", str(tmp_path / "c"))
    got = dict(re.findall(r"(\w+)=(\S+)", line))
    assert float(got["clock_mhz"]) == pytest.approx(2000, abs=1)
    assert float(got["mfma_busy_pct"]) == pytest.approx(60.0, abs=0.05)
    assert float(got["dispatch_us"]) == pytest.approx(500.0)


def test_counters_without_the_kernel_fail_loudly(tmp_path):
    _write(tmp_path / "c", [(VENDOR, "GRBM_GUI_ACTIVE", 1.0, 0, 1)])
    with pytest.raises(SystemExit):
        bench.summarize_counters("s8s8", str(tmp_path / "c"))


def test_kernel_names_match_the_committed_trace():
    """Every workload's kernel name prefix occurs in the committed kernel
    trace of the benchmark, so the summaries find the kernels that ran."""
    trace = open(os.path.join(ROOT, "profiles", "kernel_trace_qgemm_step.md")).read()
    for name, kn in bench.KERNEL_NAMES.items():
        assert kn in trace, (name, kn)


@pytest.mark.parametrize("lib,symbols", [
    ("libqgcalib.so", ["qgc_stream_read", "qgc_mfma_stream", "qgc_wall_clock_khz"]),
    ("libqgvendor.so", ["qgv_int8_gemm_search"]),
])
def test_helper_libraries_export(lib, symbols):
    path = os.path.join(ROOT, "conv_qgemm_amd", lib)
    if not os.path.exists(path):
        pytest.skip(f"{lib} is not built")
    so = ctypes.CDLL(path)
    for s in symbols:
        assert hasattr(so, s), s


def test_code_fingerprint_ignores_comments_only():
    """The counters stay attached to a kernel through comment and layout
    edits, and detach on any change of code, string literals included."""
    src = 'int f(int x) {  // add one\n  return x + 1; /* done */ }\nconst char *s = "a // b";\n'
    same = '/* header */\nint f(int x)\n{\n    return x + 1;\n}\nconst char *s = "a // b";  // literal\n'
    assert bench.code_text(src) == bench.code_text(same)
    for changed in (src.replace("x + 1", "x + 2"), src.replace('"a // b"', '"a // c"'),
                    src.replace("return", "return -")):
        assert bench.code_text(changed) != bench.code_text(src)
    assert "add one" not in bench.code_text(src) and "// b" in bench.code_text(src)

