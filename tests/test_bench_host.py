"""Host-side checks of bench.py (no GPU): the multi-GPU refusal, the rocprofv3 CSV
summariser and the traffic read-back that `roofline.traffic` comes from."""
import csv
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402

C128A = "void kvq::compress_long_kernel<(kvq::Layout)1, 128, 8, 2>(unsigned char*, long)"
C4A = "void kvq::compress_short_kernel<(kvq::Layout)1, 4, false>(unsigned char*, long)"
COPY = "__amd_rocclr_copyBuffer"


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2 and "one GPU" in r.stderr


def _write(path, header, rows):
    os.makedirs(os.path.dirname(path), exist_ok=True)
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(header)
        w.writerows(rows)


@pytest.fixture
def results(tmp_path):
    _write(str(tmp_path / "prof_trace" / "trace_kernel_stats.csv"),
           ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs", "StdDev"],
           [[C128A, 11, 0, 1227020.0, 50, 1219600, 1242440, 0], [C4A, 11, 0, 46840.0, 2, 44510, 52870, 0],
            ["some_other_kernel", 3, 0, 1000.0, 0, 900, 1100, 0]])
    _write(str(tmp_path / "prof_trace" / "trace_kernel_trace.csv"), ["Kernel_Name", "Start_Timestamp", "End_Timestamp"],
           [[C128A, 1000 * k, 1000 * k + (1300000 if k < 10 else 1227020)] for k in range(30)])
    # counters in KiB per dispatch: the 1 GiB copy reads half its bytes in FETCH_SIZE
    alg = bench.bytes_compress(16384, 128, 528)
    hdr = ["Kernel_Name", "Grid_Size", "Counter_Value"]
    _write(str(tmp_path / "pmc_fetch" / "fetch_counter_collection.csv"), hdr,
           [[COPY, 777, 524288.0], [COPY, 5, 12.0], [C128A, 16384, alg * 1.01 / 2 / 1024],
            [C4A, 4096, 1000.0]])
    _write(str(tmp_path / "pmc_write" / "write_counter_collection.csv"), hdr,
           [[COPY, 777, 1048576.0], [COPY, 5, 3.0], [C128A, 16384, 0.0], [C4A, 4096, 10.0]])
    # DRAM sectors of 32 bytes: the copy moves 1 GiB each way; C128A reads 1.01x algorithmic
    rd, wr, r128 = "TCC_EA0_RDREQ_DRAM_32B_sum", "TCC_EA0_WRREQ_WRITE_DRAM_32B_sum", "TCC_EA0_RDREQ_128B_sum"
    _write(str(tmp_path / "pmc_dram" / "dram_counter_collection.csv"), ["Kernel_Name", "Grid_Size", "Counter_Name",
                                                                        "Counter_Value"],
           [[COPY, 777, rd, (1 << 30) / 32], [COPY, 777, wr, (1 << 30) / 32], [COPY, 777, r128, (1 << 30) / 128],
            [COPY, 5, rd, 10.0], [COPY, 5, wr, 1.0], [COPY, 5, r128, 2.0],
            [C128A, 16384, rd, alg * 1.01 / 32], [C128A, 16384, wr, 0.0], [C128A, 16384, r128, alg / 128],
            [C4A, 4096, rd, 100.0], [C4A, 4096, wr, 10.0], [C4A, 4096, r128, 25.0]])
    return str(tmp_path)


def test_trace_summary_lists_named_kernels(results):
    text = bench.trace_summary(results)
    assert "compress_long<V41, ratio 128> (C128A)" in text and "1227.02" in text
    line = [ln for ln in text.splitlines() if ln.startswith("compress_long<V41, ratio 128>")][0]
    assert line.split()[-4] == "1227.02"           # after the 10 warmup launches
    assert "some_other_kernel" not in text


def test_pmc_summary_scales_by_the_copy_and_round_trips(results, tmp_path, monkeypatch):
    text = bench.pmc_summary(results)
    assert "(scale 2.0)" in text and "(scale 1.0)" in text
    assert "1.010 x algorithmic" in text
    prof = tmp_path / "pmc.txt"
    prof.write_text(text)
    monkeypatch.setattr(bench, "PROFILE", str(prof))
    t = bench.read_traffic(bench.bytes_compress(16384, 128, 528))
    assert t is not None and abs(t["ratio_to_algorithmic"] - 1.01) < 1e-6
    assert abs(t["fetch_write_scaled_bytes"] / t["bytes"] - 1.0) < 1e-6     # both counts agree
    # a kernel-source change makes the stored counters stale
    prof.write_text(text.replace(bench.kernel_source_hash(), "0" * 64))
    assert bench.read_traffic(bench.bytes_compress(16384, 128, 528)) is None



def test_all_kernels_summary_groups_by_kernel_and_grid(tmp_path):
    hdr = ["Kind", "Kernel_Name", "Start_Timestamp", "End_Timestamp", "LDS_Block_Size",
           "Workgroup_Size_X", "Grid_Size_X"]
    short4 = "void kvq::compress_short_kernel<(kvq::Layout)1, 4>(unsigned char*, long)"
    rows = [["KERNEL_DISPATCH", short4, 0, 47000, 0, 256, 4096 * 256],
            ["KERNEL_DISPATCH", short4, 0, 45000, 0, 256, 4096 * 256],
            ["KERNEL_DISPATCH", short4, 0, 1620000, 0, 256, 131072 * 256],
            ["KERNEL_DISPATCH", "__amd_rocclr_copyBuffer", 0, 5, 0, 256, 256]]
    _write(str(tmp_path / "prof_next" / "next_kernel_trace.csv"), hdr, rows)
    text = bench.all_kernels_summary(str(tmp_path))
    lines = [ln for ln in text.splitlines() if ln.startswith("compress_short_kernel<V41, 4>")]
    assert len(lines) == 2                                   # one line per grid
    assert lines[0].split()[2:6] == ["4096", "256", "0", "2"] and "46.00" in lines[0]
    assert "copyBuffer" not in text
