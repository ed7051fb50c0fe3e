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
    """Per shape, the last GEMM_PMC_REPS of its run of GEMM dispatches are
    averaged; the byte counters are scaled by the calibration copy; the figures
    follow, one column per shape."""
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    reps = bench.GEMM_PMC_REPS
    assert bench.GEMM_PMC_SHAPES == ("qkvo", "gate_up")
    kernels = ["void bitnet::gemm_mfma_kernel<128, 256, 2, 4, 2, 3, true, false>(...)",
               "void bitnet::gemm_mfma_kernel<128, 256, 1, 4, 2, 2, true, false>(...)"]
    passes = {  # per shape: the kept dispatches' counters
        "a": [{"SQ_INSTS_MFMA": 1048576, "SQ_VALU_MFMA_BUSY_CYCLES": 1048576 * 32, "SQ_INSTS_VALU": 1048576 * 7.5,
               "SQ_VALU_MFMA_COEXEC_CYCLES": 1048576 * 16},
              {"SQ_INSTS_MFMA": 2818048, "SQ_VALU_MFMA_BUSY_CYCLES": 2818048 * 32, "SQ_INSTS_VALU": 2818048 * 4,
               "SQ_VALU_MFMA_COEXEC_CYCLES": 2818048 * 8}],
        "b": [{"SQ_WAIT_INST_ANY": 400, "SQ_WAVE_CYCLES": 1000, "SQ_INSTS_LDS": 900000, "SQ_LDS_BANK_CONFLICT": 0,
               "SQ_WAIT_INST_LDS": 50, "SQ_BUSY_CYCLES": 1},
              {"SQ_WAIT_INST_ANY": 300, "SQ_WAVE_CYCLES": 1000, "SQ_INSTS_LDS": 900000, "SQ_LDS_BANK_CONFLICT": 9000,
               "SQ_WAIT_INST_LDS": 20, "SQ_BUSY_CYCLES": 1}],
        "fetch": [{"FETCH_SIZE": 14336.0}, {"FETCH_SIZE": 30000.0}],   # KiB; x2 by the calibration below
        "write": [{"WRITE_SIZE": 16384.0}, {"WRITE_SIZE": 44032.0}],   # KiB; x1
    }
    ends = [35000, 90000]
    calib = {"fetch": ("FETCH_SIZE", bench.CALIB_COPY_BYTES / 2 / 1024), "write": ("WRITE_SIZE",
                                                                                  bench.CALIB_COPY_BYTES / 1024)}
    dirs = []
    for p, per_shape in passes.items():
        d = tmp_path / p
        d.mkdir()
        rows = []
        if p in calib:
            rows += [[1, "__amd_rocclr_copyBuffer", calib[p][0], calib[p][1], 0, 1]]
        did = 10
        for s, counters in enumerate(per_shape):
            # warm-up dispatches with different values, then the kept ones
            for i in range(5):
                rows += _counter_rows(kernels[s], did, {k: 0 for k in counters}, end=99000)
                did += 1
            for i in range(reps):
                rows += _counter_rows(kernels[s], did, counters, end=ends[s])
                did += 1
        _write_csv(d / "run_counter_collection.csv", header, rows)
        dirs.append(str(d))
    out = tmp_path / "gemm.md"
    monkeypatch.setattr(bench, "GEMM_PMC_FILE", str(out))
    bench.summarize_gemm_pmc(dirs)
    text = out.read_text()
    assert "| workgroups | 256 of 8 waves | 688 of 4 waves |" in text
    assert "| dispatch duration (profiled) | 35.00 µs | 90.00 µs |" in text
    f0 = 1048576 * 32 / (35000e-9 * 2.4e9 * 1024)
    f1 = 2818048 * 32 / (90000e-9 * 2.4e9 * 1024)
    assert f"| MFMA busy / (duration × 2.4 GHz × 1024 SIMDs) | {f0:.3f} | {f1:.3f} |" in text
    assert "| VALU instructions per MFMA | 7.50 | 4.00 |" in text
    assert "| MFMA cycles with VALU co-issued (COEXEC / MFMA busy) | 0.500 | 0.250 |" in text
    assert "| LDS bank-conflict cycles per LDS instruction | 0.00 | 0.01 |" in text
    assert "| SQ_WAIT_INST_ANY / SQ_WAVE_CYCLES | 0.400 | 0.300 |" in text
    hbm0 = 14336 * 1024 * 2 + 16384 * 1024
    hbm1 = 30000 * 1024 * 2 + 44032 * 1024
    assert f"| HBM bytes (FETCH_SIZE × 2.000 + WRITE_SIZE × 1.000) | {hbm0:.4g} " in text
    assert f"| {hbm1:.4g} (" in text


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


def test_step_plan_runs_exactly_the_asked_steps():
    """The headline's replay plan covers exactly n steps, on consecutive weight
    copies, whatever the starting step and the number of copies."""
    for copies in (1, 2, 11):
        for start in (0, 3, 11, 25):
            for n in (0, 1, 5, 20, 22, 2200):
                plan, nxt = bench.step_plan(start, n, copies)
                steps = []
                i = start
                for c in plan:
                    if c is None:
                        assert i % copies == 0
                        steps += list(range(copies))
                        i += copies
                    else:
                        assert c == i % copies
                        steps.append(c)
                        i += 1
                assert len(steps) == n and nxt == start + n
                assert steps == [(start + j) % copies for j in range(n)]
    # whole rotations are one replay each
    assert bench.step_plan(0, 22, 11) == ([None, None], 22)
    assert bench.step_plan(5, 20, 11)[0] == [5, 6, 7, 8, 9, 10, None, 0, 1, 2]


def test_percentiles():
    st = bench.pstats([1e-6 * v for v in range(1, 12)])      # 1 .. 11 us
    assert st["n"] == 11 and abs(st["median"] - 6.0) < 1e-9
    assert abs(st["p10"] - 2.0) < 1e-9 and abs(st["p90"] - 10.0) < 1e-9


def test_host_facts():
    f = bench.host_facts()
    assert f["nproc"] == os.cpu_count() and f["usable_cpus"] >= 1 and f["cpu_model"]


def test_summarize_small_pmc(tmp_path, monkeypatch):
    """Per case, the last SMALL_PMC_REPS of its dispatches are averaged; byte
    counters are scaled by the calibration copy; the ratio to the algorithmic
    bytes and the wait fraction follow."""
    monkeypatch.setattr(bench, "SMALL_PMC_WARM", 2)
    monkeypatch.setattr(bench, "SMALL_PMC_REPS", 3)
    monkeypatch.setattr(bench, "SMALL_PMC_FILE", str(tmp_path / "small.md"))
    cases = bench.small_pmc_cases()
    header = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value", "Start_Timestamp", "End_Timestamp"]
    dirs = []
    for p, counters in bench.SMALL_PMC_PASSES.items():
        d = tmp_path / p
        d.mkdir()
        rows = []
        if p in ("fetch", "write"):
            cn = "FETCH_SIZE" if p == "fetch" else "WRITE_SIZE"
            rows.append([1, "__amd_rocclr_copyBuffer", cn, bench.CALIB_COPY_BYTES / 1024 / (2 if p == "fetch" else 1), 0, 1])
        did = 10
        for c, (tag, kind, M, N, K, j) in enumerate(cases):
            name = "void gemv_stream_kernel<1, 4>" if kind == "gemv" else "void gemm_skinny_lds_kernel<1, 1, 8, false>"
            algo = bench.gemv_bytes(M, N, K) if kind == "gemv" else bench.gemm_bytes(M, N, K)
            for i in range(5):
                kept = i >= 2
                vals = {"SQ_WAIT_INST_ANY": 300 if kept else 0, "SQ_WAVE_CYCLES": 1000, "SQ_BUSY_CYCLES": 1,
                        "SQ_WAVES": 480, "GRBM_GUI_ACTIVE": 1,
                        "FETCH_SIZE": (algo / 2 / 1024) if kept else 0.0, "WRITE_SIZE": 0.0}
                for cn in counters.split():
                    rows.append([did, name, cn, vals[cn], 0, 4000])
                did += 1
        _write_csv(d / "run_counter_collection.csv", header, rows)
        dirs.append(str(d))
    bench.summarize_small_pmc(dirs)
    text = (tmp_path / "small.md").read_text()
    # FETCH_SIZE x 2 = algorithmic bytes: ratio 1.000; 4 us dispatches; wait fraction 0.3
    tag, kind, M, N, K, j = cases[0]
    assert f"| {tag} | `gemv_stream_kernel<1, 4>` | 4.00 | " in text
    assert "| 1.000 | " in text and "| 0.300 | 480 |" in text
