"""bench.py's host logic on a machine without a GPU: the one-GPU guard,
workload lookup, the comment-blind source digest that keeps stored counters
honest, the calibration arithmetic of the HBM-traffic summary, and the shape
of the CPU-baseline record."""
import os
import shutil
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)
import bench  # noqa: E402
from io_aware_tiled_08_amd import workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, cwd=ROOT, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_every_workload_has_a_kernel_key():
    names = (list(W.WORKLOADS) + list(W.CACHE_WORKLOADS) + list(W.FP8_WORKLOADS)
             + list(W.BWD_WORKLOADS))
    for name in names:
        w, key = bench.workload_by_name(name)
        assert w.name == name
        assert key in bench.KERNEL_SOURCES and key in bench.KERNEL_NAME_PATTERN
    assert bench.workload_by_name("headline_f16_d128")[1] == "f16"
    assert bench.workload_by_name("decode_long_bf16")[1] == "kvcache"
    assert bench.workload_by_name("headline_bwd_f16_d128")[1] == "bwd"
    with pytest.raises(SystemExit):
        bench.workload_by_name("no_such_workload")


def test_digest_ignores_comments_but_not_code(tmp_path, monkeypatch):
    src = tmp_path / "csrc"
    shutil.copytree(bench._CSRC, src)
    monkeypatch.setattr(bench, "_CSRC", str(src))
    base = bench.kernel_source_digest("bwd")
    p = src / "fa_bwd.hip"
    text = p.read_text()
    p.write_text("// a new comment line\n" + text.replace("namespace fa {", "namespace fa {  /* x */\n\n", 1))
    assert bench.kernel_source_digest("bwd") == base
    p.write_text(text.replace("constexpr int kDkvQ = 32;", "constexpr int kDkvQ = 64;"))
    assert bench.kernel_source_digest("bwd") != base
    assert bench.kernel_source_digest("f16") != base


def _pmc_csv(path, counter, rows):
    with open(path, "w") as f:
        f.write("Kernel_Name,Counter_Name,Counter_Value\n")
        for name, value in rows:
            f.write(f"{name},{counter},{value}\n")


def test_traffic_summary_calibrates_against_the_copy(tmp_path, monkeypatch):
    """Five calls of three kernels each; the 512 MiB calibration copies read
    as a little over half their size for FETCH_SIZE (as the counter reports
    for a device copy) and as their size for WRITE_SIZE; a small copy and an
    unrelated kernel are ignored."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    copy_kib = bench.COPY_BYTES / 1024
    fetch = [("bwd_prep_kernel", 10.0), ("bwd_dkdv_kernel", 1000.0), ("bwd_dq_kernel", 500.0)] * 5
    fetch += [("elementwise_copy", copy_kib / 2 + 16.0)] * 3 + [("elementwise_copy", 4.0), ("other", 9e9)]
    write = [("bwd_prep_kernel", 1.0), ("bwd_dkdv_kernel", 100.0), ("bwd_dq_kernel", 50.0)] * 5
    write += [("elementwise_copy", copy_kib)] * 3
    _pmc_csv(tmp_path / "f.csv", "FETCH_SIZE", fetch)
    _pmc_csv(tmp_path / "w.csv", "WRITE_SIZE", write)
    path = bench.summarize_traffic(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                   "headline_bwd_f16_d128")
    expect = 1510.0 * 1024 * copy_kib / (copy_kib / 2 + 16.0) + 151.0 * 1024
    text = open(path).read()
    assert f"hbm_bytes_per_launch: {expect:.0f}" in text
    assert bench.measured_traffic("headline_bwd_f16_d128", "bwd") == pytest.approx(expect)
    # a stored summary whose source hash no longer matches is ignored
    open(path, "w").write(text.replace(bench.kernel_source_digest("bwd"), "0" * 64))
    assert bench.measured_traffic("headline_bwd_f16_d128", "bwd") is None


def test_cpu_baseline_record():
    w = W.WORKLOADS["single_head_f32"]
    q, k, v = W.workload_inputs(w)
    rec = bench.cpu_baseline(w, q, k, v, 0.2)
    assert rec["kind"] == "oracle" and rec["unit"] == "TFLOP/s"
    assert rec["value"] > 0 and rec["cores"] >= 1 and w.name in rec["sample"]


def test_cpu_baseline_counts_the_threads_it_used():
    """The record names the threads of the pool (one per core this process may
    use, at most 16), the cores the host gives it, and the CPU model; the
    whole small workload fits the budget."""
    w = W.WORKLOADS["single_head_f32"]
    q, k, v = W.workload_inputs(w)
    rec = bench.cpu_baseline(w, q, k, v, 5.0)
    cores = len(os.sched_getaffinity(0))
    assert rec["cores"] == min(cores, 16) and rec["host_cores"] == cores
    assert isinstance(rec["cpu_model"], str)
    assert rec["sample"].startswith(f"{w.N} of {w.N} query rows")


def test_cpu_baseline_reports_the_difference_from_given_outputs():
    """With the GPU's outputs handed in, the record gives max |O - oracle| and
    max |LSE - oracle| over the rows it computed: zero for the oracle's own
    outputs, and exactly a planted offset otherwise."""
    import numpy as np

    import oracle
    w = W.WORKLOADS["single_head_f32"]
    q, k, v = W.workload_inputs(w)
    O, L = oracle.attention_forward(q, k, v, w.scale, w.causal)
    rec = bench.cpu_baseline(w, q, k, v, 5.0, gpu_out=(O.copy(), L.copy()))
    assert rec["max_abs_err"] == {"O": 0.0, "LSE": 0.0, "rows": w.N}
    O2, L2 = O.copy(), L.copy()
    O2[0, 0, 300, 5] += 0.25
    L2[0, 0, 7] -= 0.125
    rec = bench.cpu_baseline(w, q, k, v, 5.0, gpu_out=(O2, L2))
    assert rec["max_abs_err"]["O"] == pytest.approx(0.25, abs=1e-12)
    assert rec["max_abs_err"]["LSE"] == pytest.approx(0.125, abs=1e-12)
    assert rec["rows"] == w.N and rec["seconds"] > 0
    assert "max_abs_err" not in bench.cpu_baseline(w, q, k, v, 0.1)
    assert np.isfinite(rec["value"])


def test_all_configs_table():
    """One row per configuration, with compulsory and counter GB/s over the
    kernel time, the oracle differences and the baseline's seconds."""
    rec = {"value": 1200.0, "config": {"workload": "headline_f16_d128"},
           "roofline": {"kernel_ms": 0.25, "compulsory_bytes": 1e8, "traffic": 2e8, "frac": 0.477},
           "cpu_baseline": {"seconds": 1.25, "cores": 16,
                            "max_abs_err": {"O": 1e-4, "LSE": 2e-5, "rows": 4096}}}
    text = bench.format_all_configs([("C3 (headline)", rec)], 100, 30.0)
    row = [x for x in text.splitlines() if x.startswith("| C3")][0]
    assert "| 1200.0 | 47.7% |" in row
    assert "400 (5.0%)" in row and "800 (10.0%)" in row  # 1e8 and 2e8 bytes in 0.25 ms
    assert "1.00e-04 / 2.00e-05 (4096)" in row and "1.2 (16)" in row
    assert "--all-configs --steps 100 --cpu-budget 30" in text
    assert [c[1] for c in bench.ALL_CONFIGS] == [
        "single_head_f32", "batch_f16_d64", "batch_f16_d64_causal", "headline_f16_d128",
        "rescale_stress_bf16", "long_context_bf16"]


def test_oracle_pool_stops_starting_units_after_the_budget():
    import time as _t
    seen = []

    def run(u):
        seen.append(u)
        _t.sleep(0.05)
        return 1.0

    total, n, el, workers = bench.run_oracle_pool(range(10000), run, 0.2)
    assert n == total == len(seen) and n < 10000
    assert el < 5.0
    # at least one unit, even with no budget
    total, n, _, _ = bench.run_oracle_pool(range(5), run, 0.0)
    assert n >= 1


def test_trace_summary_averages_the_timed_dispatches(tmp_path, monkeypatch):
    """Dispatches are counted per kernel: the first (settle calls + warm-up)
    are skipped, the next `steps` are the timed region."""
    import json
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    name = "_ZN2fa_fwd_f16_persistent_kernel"
    with open(d / "trace_kernel_stats.csv", "w") as f:
        f.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        f.write(f'"{name}",30,0,150,100,100,300,10\n')
    with open(d / "trace_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for i in range(30):  # 10 settle + 5 warm-up at 100 ns, 10 timed at 200 ns, 5 more at 300 ns
            dur = 100 if i < 15 else (200 if i < 25 else 300)
            f.write(f"{name},{1000 * i},{1000 * i + dur}\n")
    log = tmp_path / "bench.log"
    rec = {"value": 1.0, "unit": "TFLOP/s", "steps": 10, "warmup": 5,
           "clock_settle": {"calls": 10},
           "roofline": {"kernel_ms": 0.0002, "frac": 0.5, "peak": 2.0, "unit": "TFLOP/s"}}
    log.write_text("noise\n" + json.dumps(rec) + "\n")
    path = bench.summarize_trace(str(tmp_path / "trace"), str(log), "headline_f16_d128")
    text = open(path).read()
    assert "200 ns over 10 dispatches" in text
    assert "event average = 1.000" in text


def test_counter_summary_reads_units_and_per_tile_counts(tmp_path, monkeypatch):
    """GRBM_GUI_ACTIVE is divided by the 8 XCDs, the matrix-busy cycles by the
    1024 SIMDs, quad-cycle wait counters by quad-cycle wave cycles, and the
    forward's instruction counts by its wave-tiles (32 rows x 128 keys)."""
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    name = "_ZN2fa_fwd_f16_persistent_kernel"
    w = W.WORKLOADS["headline_f16_d128"]
    n_wt = w.B * w.H * (w.N // 32) * (w.N // 128)
    length = 400000
    values = {"GRBM_GUI_ACTIVE": 8 * length, "SQ_VALU_MFMA_BUSY_CYCLES": 0.5 * length * 1024,
              "SQ_VALU_MFMA_COEXEC_CYCLES": 0.25 * length * 1024, "SQ_WAVE_CYCLES": 1000.0,
              "SQ_WAIT_INST_LDS": 100.0, "SQ_INSTS_VALU": 300.0 * n_wt, "SQ_INSTS_MFMA": 80.0 * n_wt,
              "SQ_ACTIVE_INST_VALU": 300.0 * n_wt}
    paths = []
    for i, chunk in enumerate((list(values)[:3], list(values)[3:6], list(values)[6:])):
        p = tmp_path / f"p{i}.csv"
        with open(p, "w") as f:
            f.write("Kernel_Name,Counter_Name,Counter_Value\n")
            for c in chunk:
                for _ in range(2):
                    f.write(f"{name},{c},{values[c]}\n")
                f.write(f"other_kernel,{c},1\n")
        paths.append(str(p))
    text = open(bench.summarize_counters(paths, "headline_f16_d128")).read()
    assert "busy length (GRBM_GUI_ACTIVE / 8): 400000 cycles" in text
    assert "matrix pipe busy per SIMD over that length: 50.0%" in text
    assert "while the matrix pipe is busy / matrix busy: 50.0%" in text
    assert "waiting to issue an LDS instruction (SQ_WAIT_INST_LDS / SQ_WAVE_CYCLES): 10.0%" in text
    assert "cycles per vector instruction (4 x SQ_ACTIVE_INST_VALU / SQ_INSTS_VALU): 4.00" in text
    assert "vector (not MFMA) 220.0, MFMA 80.0" in text
    assert "other_kernel" not in text


def test_trace_summary_skips_the_untimed_graph_replay(tmp_path, monkeypatch):
    """With --graph the timed replay follows one untimed replay of the same
    `steps` dispatches, so the timed region starts `steps` dispatches later."""
    import json
    monkeypatch.setattr(bench, "PROFILES", str(tmp_path / "profiles"))
    d = tmp_path / "trace" / "host"
    d.mkdir(parents=True)
    name = "_ZN2fa_fwd_f32_q4_kernel"
    with open(d / "trace_kernel_stats.csv", "w") as f:
        f.write('"Name","Calls","TotalDurationNs","AverageNs","Percentage","MinNs","MaxNs","StdDev"\n')
        f.write(f'"{name}",25,0,150,100,100,300,10\n')
    with open(d / "trace_kernel_trace.csv", "w") as f:
        f.write("Kernel_Name,Start_Timestamp,End_Timestamp\n")
        for i in range(25):  # 5 warm-up + 10 untimed replay at 100 ns, 10 timed at 200 ns
            dur = 100 if i < 15 else 200
            f.write(f"{name},{1000 * i},{1000 * i + dur}\n")
    log = tmp_path / "bench.log"
    rec = {"value": 1.0, "unit": "TFLOP/s", "steps": 10, "warmup": 5, "launch": "hip_graph",
           "clock_settle": {"calls": 0},
           "roofline": {"kernel_ms": 0.0002, "frac": 0.5, "peak": 2.0, "unit": "TFLOP/s"}}
    log.write_text(json.dumps(rec) + "\n")
    text = open(bench.summarize_trace(str(tmp_path / "trace"), str(log), "single_head_f32")).read()
    assert "200 ns over 10 dispatches" in text
    assert "--graph" in text and "captured HIP graph" in text
