"""Host logic of bench.py, on the CPU: the algorithmic byte counts, the
one-GPU contract, and the rocprofv3 summarisers on small synthetic CSV folders
(the column names rocprofv3 writes, values chosen so every figure is known)."""
import csv
import gzip
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402


def test_algorithmic_bytes():
    # packed W (N*K/4) + bf16 scale_wt (2N) + bf16 x (2MK) + bf16 out (2MN)
    assert bench.gemv_bytes(1, 128256, 2560) == 128256 * 640 + 2 * 128256 + 2 * 2560 + 2 * 128256
    assert bench.gemv_bytes(1, 128256, 2560) == 82601984
    # packed W + scale_wt + int8 x (MK) + bf16 scale_act (2M) + bf16 out (2MN)
    assert bench.gemm_bytes(2048, 4096, 4096) == 4096 * 1024 + 2 * 4096 + 2048 * 4096 + 2 * 2048 + 2 * 2048 * 4096
    assert bench.gemm_bytes(2048, 4096, 4096) == 29372416
    # int8 W + fp32 scale + bf16 x + fp32 y
    assert bench.w8a16_bytes(16, 4096, 4096) == 4096 * 4096 + 4 * 4096 + 2 * 16 * 4096 + 4 * 16 * 4096


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, cwd=ROOT, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def _write_csv(path, header, rows, gz=False):
    opener = gzip.open if gz else open
    with opener(path, "wt", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_summarize_trace_reads_plain_and_gzipped_csv(tmp_path, capsys):
    _write_csv(tmp_path / "bench_kernel_stats.csv",
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [["gemv_stream_kernel", 3, 45000, 15000, 90.0, 14000, 16000],
                ["gemm_mfma_kernel", 1, 5000, 5000, 10.0, 5000, 5000]])
    trace = [["gemv_stream_kernel", 128256, 100, 14100], ["gemv_stream_kernel", 128256, 200, 16200],
             ["gemv_stream_kernel", 20480, 300, 4300], ["gemm_mfma_kernel", 131072, 0, 5000]]
    _write_csv(tmp_path / "bench_kernel_trace.csv.gz", ["Kernel_Name", "Grid_Size", "Start_Timestamp", "End_Timestamp"],
               trace, gz=True)
    bench.summarize_trace(str(tmp_path))
    text = capsys.readouterr().out
    assert "| `gemv_stream_kernel` | 3 | 0.045 | 15.000 | 14.000 | 16.000 | 90.00 |" in text
    # the per-grid table splits one kernel by launch grid: two launches of 14 and 16 us at 128256 threads
    assert "| `gemv_stream_kernel` | 128256 | 2 | 15.000 | 14.000 | 16.000 |" in text
    assert "| `gemv_stream_kernel` | 20480 | 1 | 4.000 | 4.000 | 4.000 |" in text


def _counter_rows(kernel, dispatch, counters, start=0, end=35000):
    return [[dispatch, kernel, name, value, start, end] for name, value in counters.items()]


def test_summarize_gemm_pmc(tmp_path, monkeypatch):
    """The last GEMM_PMC_REPS GEMM dispatches of each pass are averaged; the byte
    counters are scaled by the calibration copy; the figures follow."""
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    reps = bench.GEMM_PMC_REPS
    passes = {
        "a": {"SQ_INSTS_MFMA": 1048576, "SQ_VALU_MFMA_BUSY_CYCLES": 1048576 * 32, "SQ_INSTS_VALU": 1048576 * 7.5,
              "SQ_VALU_MFMA_COEXEC_CYCLES": 1048576 * 16},
        "b": {"SQ_WAIT_INST_ANY": 400, "SQ_WAVE_CYCLES": 1000, "SQ_INSTS_LDS": 900000, "SQ_LDS_BANK_CONFLICT": 0,
              "SQ_WAIT_INST_LDS": 50, "SQ_BUSY_CYCLES": 1},
        "fetch": {"FETCH_SIZE": 14336.0},   # KiB; x2 by the calibration below
        "write": {"WRITE_SIZE": 16384.0},   # KiB; x1
    }
    calib = {"fetch": ("FETCH_SIZE", bench.CALIB_COPY_BYTES / 2 / 1024), "write": ("WRITE_SIZE",
                                                                                  bench.CALIB_COPY_BYTES / 1024)}
    dirs = []
    for p, counters in passes.items():
        d = tmp_path / p
        d.mkdir()
        rows = []
        if p in calib:
            rows += [[1, "__amd_rocclr_copyBuffer", calib[p][0], calib[p][1], 0, 1]]
        # warm-up dispatches with different values, then the kept ones
        for i in range(5):
            rows += _counter_rows("void gemm_mfma_kernel<...>", 10 + i, {k: 0 for k in counters}, end=99000)
        for i in range(reps):
            rows += _counter_rows("void gemm_mfma_kernel<...>", 100 + i, counters)
        _write_csv(d / "run_counter_collection.csv", header, rows)
        dirs.append(str(d))
    out = tmp_path / "gemm.md"
    monkeypatch.setattr(bench, "GEMM_PMC_FILE", str(out))
    bench.summarize_gemm_pmc(dirs)
    text = out.read_text()
    assert "(`gemm_mfma_kernel<...>`, 256 workgroups" in text
    assert "| dispatch duration (profiled) | 35.00 µs |" in text
    frac = 1048576 * 32 / (35000e-9 * 2.4e9 * 1024)
    assert f"| MFMA busy / (duration × 2.4 GHz × 1024 SIMDs) | {frac:.3f} |" in text
    assert "| VALU instructions per MFMA | 7.50 |" in text
    assert "| MFMA cycles with VALU co-issued (COEXEC / MFMA busy) | 0.500 |" in text
    assert "| SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES | 0.400 |" in text
    hbm = 14336 * 1024 * 2 + 16384 * 1024
    assert f"| HBM bytes (FETCH_SIZE × 2.000 + WRITE_SIZE × 1.000) | {hbm:.4g} " in text


def test_summarize_gemm_pmc_needs_enough_dispatches(tmp_path):
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    dirs = []
    for p in bench.GEMM_PMC_PASSES:
        d = tmp_path / p
        d.mkdir()
        _write_csv(d / "run_counter_collection.csv", header,
                   _counter_rows("void gemm_mfma_kernel<...>", 1, {"SQ_INSTS_MFMA": 1}))
        dirs.append(str(d))
    with pytest.raises(SystemExit):
        bench.summarize_gemm_pmc(dirs)


def test_gemv_scaling_fit():
    """The line fit recovers a known fixed cost and rate, and ignores the small-N rows."""
    K = 2560
    rows = []
    for N in bench.GEMV_SCALING_N:
        mb = N * K / 4 / 1e6
        t_us = 3.5 + mb / 6.7 if N >= bench.GEMV_SCALING_FIT_MIN_N else 100.0  # small N: off the line
        rows.append((N, mb, t_us * 1e-6))
    fixed, rate = bench.scaling_fit(rows)
    assert abs(fixed - 3.5) < 1e-9 and abs(rate - 6.7) < 1e-9
