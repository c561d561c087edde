"""Host-only parts of bench.py (no GPU): the one-GPU refusal, the HBM-traffic
calibration arithmetic over rocprofv3 counter CSVs, and the kernel-stats
summary.  The CSVs are small synthetic files in rocprofv3's column layout."""
import csv
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_counters(path, counter, rows):
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for d, row in enumerate(rows):
            kernel, value = row[0], row[1]
            grid = row[2] if len(row) > 2 else 65536
            # two counter rows per dispatch (as for a counter summed over blocks)
            for half in (0.25, 0.75):
                w.writerow({"Dispatch_Id": d, "Kernel_Name": kernel + "(int, float*)", "Grid_Size": grid,
                            "Counter_Name": counter, "Counter_Value": value * half})


def _dma_calibration(counter, factor):
    """The one-tile DMA calibration launches (grid of 256 work-items), three
    of each GEMM, whose counters read 1/factor of the known bytes."""
    rows = []
    for api, (kname, rbytes, wbytes) in bench.DMA_CALIB.items():
        b = rbytes if counter == "FETCH_SIZE" else wbytes
        rows += [(kname.replace("*", "0"), b / 1024.0 / factor, 256)] * 3
    return rows


def test_traffic_calibration(tmp_path):
    mib = 64
    n = mib * (1 << 20) // 2
    # the streaming calibration kernel reads 4n and writes 2n bytes; its
    # counters read half the fetched bytes (factor 2) and all the written ones
    # (factor 1).  The DMA path's one-tile launches read a third of the
    # fetched bytes (factor 3) and all the written ones: the GEMMs take those.
    cal_f, cal_w = 4.0 * n / 1024 / 2, 2.0 * n / 1024
    main, split, fix = "dmpq::gemm_fp4_dma_kernel<1, 0>", "dmpq::gemm_fp4_split_kernel", \
        "dmpq::gemm_f32_fixup_kernel<1, 0, 3>"
    fetch = [(bench.CALIB_KERNEL, cal_f)] * 3 + _dma_calibration("FETCH_SIZE", 3.0) + \
        [(main, 1000.0), (split, 100.0), (fix, 50.0), (main, 1200.0)]
    write = [(bench.CALIB_KERNEL, cal_w)] * 3 + _dma_calibration("WRITE_SIZE", 1.0) + \
        [(main, 300.0), (split, 40.0), (fix, 20.0), (main, 340.0)]
    fcsv, wcsv, out = tmp_path / "f.csv", tmp_path / "w.csv", tmp_path / "t.json"
    _write_counters(fcsv, "FETCH_SIZE", fetch)
    _write_counters(wcsv, "WRITE_SIZE", write)
    bench.summarize_traffic(str(fcsv), str(wcsv), str(out), f"x --calibrate-mib {mib} y")
    rec = json.loads(out.read_text())
    assert rec["calibration"]["fetch_factor"] == pytest.approx(2.0)
    assert rec["calibration"]["write_factor"] == pytest.approx(1.0)
    assert rec["calibration_dma"]["qgemm_nvfp4"]["fetch_factor"] == pytest.approx(3.0)
    r = rec["qgemm_nvfp4"]
    assert r["calls"] == 2 and r["dispatches"] == 4  # two whole-tile launches, split + fixup once
    assert r["fetch_bytes_per_launch"] == round(1024 * 3.0 * (1000 + 100 + 50 + 1200) / 2)
    assert r["write_bytes_per_launch"] == round(1024 * 1.0 * (300 + 40 + 20 + 340) / 2)
    assert r["sources_sha256"] == bench.sources_sha256("qgemm_nvfp4")
    assert r["traffic_over_algorithmic"] == round(
        r["bytes_per_launch"] / bench.gemm_algorithmic_bytes("qgemm_nvfp4"), 3)
    assert "qgemm_int8" not in rec  # no dispatches of it in the files


def test_traffic_needs_three_calibration_dispatches(tmp_path):
    fcsv, wcsv = tmp_path / "f.csv", tmp_path / "w.csv"
    _write_counters(fcsv, "FETCH_SIZE", [(bench.CALIB_KERNEL, 1.0)] * 2)
    _write_counters(wcsv, "WRITE_SIZE", [(bench.CALIB_KERNEL, 1.0)] * 2)
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(fcsv), str(wcsv), str(tmp_path / "t.json"), "--calibrate-mib 1")
    # the DMA calibration launches are required too
    _write_counters(fcsv, "FETCH_SIZE", [(bench.CALIB_KERNEL, 1.0)] * 3)
    _write_counters(wcsv, "WRITE_SIZE", [(bench.CALIB_KERNEL, 1.0)] * 3)
    with pytest.raises(SystemExit):
        bench.summarize_traffic(str(fcsv), str(wcsv), str(tmp_path / "t.json"), "--calibrate-mib 1")


def test_algorithmic_bytes_closed_form():
    # the 5B shapes at 17776 tokens: operands once (INT8: K bytes per row plus a
    # 4-byte scale) and the bf16 output once, averaged over the four linears
    M = 17776
    shapes = [(9216, 3072), (3072, 3072), (12288, 3072), (3072, 12288)]
    want = sum((M + N) * (K + 4) + 2.0 * M * N for N, K in shapes) / 4
    assert bench.gemm_algorithmic_bytes("qgemm_int8") == pytest.approx(want)


def test_stats_summary(tmp_path):
    rows = [("void dmpq::gemm_fp4_dma_kernel<1, 0>(unsigned char const*)", 8, 700e3, 40.0),
            ("dmpq::gemm_fp4_split_kernel(unsigned char const*)", 6, 50e3, 2.0),
            ("void dmpq::gemm_f32_fixup_kernel<1, 0, 3>(float const*)", 6, 10e3, 0.5),
            ("at::native::vectorized_elementwise_kernel<4>(int)", 3, 5e3, 1.0)]
    path = tmp_path / "s.csv"
    with open(path, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs", "Percentage"])
        w.writeheader()
        for name, calls, avg, pct in rows:
            w.writerow({"Name": name, "Calls": calls, "AverageNs": avg, "MinNs": avg, "MaxNs": avg,
                        "Percentage": pct})
    out = tmp_path / "s.md"
    bench.summarize_stats(str(path), str(out), "the command")
    md = out.read_text()
    assert "`dmpq::gemm_fp4_dma_kernel<1, 0>` | 8 | 700.0" in md
    assert "Other kernels (torch input generation, setup): 1.0%" in md
    # per call: (8 * 700 + 6 * 50 + 6 * 10) / 8 us
    assert f"| qgemm_nvfp4 | 8 | 3 | {(8 * 700 + 6 * 50 + 6 * 10) / 8:.1f} |" in md
    assert "the command" in md


def test_counter_summary(tmp_path):
    """Two counter runs of two dispatches each: cycles per XCD, clock, MFMA
    busy share and the ratios follow the stated definitions."""
    def write(path, counters):
        with open(path, "w", newline="") as f:
            w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Grid_Size", "Counter_Name",
                                              "Counter_Value", "Start_Timestamp", "End_Timestamp"])
            w.writeheader()
            for d in range(2):
                for c, v in counters.items():
                    w.writerow({"Dispatch_Id": d, "Kernel_Name": "void dmpq::gemm_i8_dma_kernel<1, 0>(int)",
                                "Grid_Size": 65536, "Counter_Name": c, "Counter_Value": v,
                                "Start_Timestamp": 1000, "End_Timestamp": 1000 + 500000})
                # a one-workgroup calibration dispatch is ignored
                w.writerow({"Dispatch_Id": 9, "Kernel_Name": "void dmpq::gemm_i8_dma_kernel<1, 0>(int)",
                            "Grid_Size": 256, "Counter_Name": "GRBM_GUI_ACTIVE", "Counter_Value": 1,
                            "Start_Timestamp": 0, "End_Timestamp": 1})
    cycles = 900000.0   # per XCD over 500 us: 1.8 GHz
    a, b, out = tmp_path / "a.csv", tmp_path / "b.csv", tmp_path / "c.md"
    write(a, {"GRBM_GUI_ACTIVE": 8 * cycles, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * cycles * 256 * 4,
              "SQ_INSTS_VALU": 300.0, "SQ_INSTS_MFMA": 100.0, "SQ_WAIT_INST_ANY": 25.0,
              "SQ_WAVE_CYCLES": 100.0})
    write(b, {"SQ_LDS_BANK_CONFLICT": 40.0, "SQ_ACTIVE_INST_LDS": 400.0})
    res = bench.summarize_counters(str(out), [str(a), str(b)], "cmd")
    r = res["dmpq::gemm_i8_dma_kernel<1, 0>"]
    assert r["dispatches"] == 2
    assert r["clock_GHz"] == pytest.approx(1.8)
    assert r["mfma_busy"] == pytest.approx(0.5)
    assert r["valu_per_mfma"] == pytest.approx(3.0)
    assert r["wait_share"] == pytest.approx(0.25)
    assert r["lds_conflict_per_active"] == pytest.approx(0.1)
    assert "| `dmpq::gemm_i8_dma_kernel<1, 0>` | 2 | 500.0 | 1.80 | 50.0% | 3.00 | 25.0% |" in out.read_text()
