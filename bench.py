"""Benchmark of the gfx950 FlashAttention forward pass on one GPU.

One step = one forward pass (scores, online softmax, P V, O and LSE written)
over the whole workload, inputs already resident in HBM.  Prints one JSON
line: throughput in TFLOP/s (4*B*H*N^2*d matrix FLOPs per step, halved under
the causal mask), the roofline of the kernel against the MI355X dense MFMA
peak, and the fp64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]

Counter workflow (HBM traffic per launch, rocprofv3 on the GPU host):

    rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/fetch -o fetch -- \\
        python3 bench.py --steps 5 --warmup 1 --settle 0 --dist 0 --cpu-budget 0 --copy-calibration
    rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/write -o write -- \\
        python3 bench.py --steps 5 --warmup 1 --settle 0 --dist 0 --cpu-budget 0 --copy-calibration
    python3 bench.py --summarize-traffic OUT/fetch/fetch_counter_collection.csv \\
        OUT/write/write_counter_collection.csv

--copy-calibration adds device-to-device copies of a known size after the
timed region; the counters of those copies turn FETCH_SIZE / WRITE_SIZE into
bytes (the factor is reported).  --summarize-traffic writes
profiles/traffic_<workload>.md, which later runs read back for the roofline's
"traffic" figure while the kernel source is unchanged.
"""
import argparse
import csv
import hashlib
import json
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
MFMA_PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3, "fp8_e4m3": 5033.2}
HBM_PEAK_GBPS = 8000.0
PEAK_CLOCK_MHZ = 2400.0  # the engine clock the published MFMA peaks are quoted at
_CSRC = os.path.join(ROOT, "io_aware_tiled_08_amd", "csrc")
# Source files each kernel is compiled from (its .hip and the headers it includes).
KERNEL_SOURCES = {
    "f16": ("fa_fwd_f16.hip", "fa_fwd_f16_ks.hip", "fa_f16_common.h", "fa_device.h"),
    "bf16": ("fa_fwd_f16.hip", "fa_fwd_f16_ks.hip", "fa_f16_common.h", "fa_device.h"),
    "f32": ("fa_fwd_f32.hip", "fa_device.h"),
    "kvcache": ("fa_fwd_kvcache.hip", "fa_f16_common.h", "fa_device.h"),
    "fp8": ("fa_fwd_fp8.hip", "fa_f16_common.h", "fa_device.h"),
    "bwd": ("fa_bwd.hip", "fa_f16_common.h", "fa_device.h"),
}
# (dominant kernel, every kernel of one call) name patterns in rocprofv3 output
KERNEL_NAME_PATTERN = {"f16": ("fwd_f16_", "fwd_f16_"),
                       "bf16": ("fwd_f16_", "fwd_f16_"),
                       "f32": ("fwd_f32_", "fwd_f32_"),
                       "kvcache": ("kvcache_fwd_kernel", "kvcache_"),
                       "fp8": ("fwd_fp8_kernel", "fwd_fp8_kernel"),
                       "bwd": ("bwd_dkdv_kernel", "bwd_")}
PROFILES = os.path.join(ROOT, "profiles")
COPY_BYTES = 512 << 20  # one calibration copy: 512 MiB read + 512 MiB written
COPY_REPS = 3
SETTLE_S = 1.5  # untimed calls before the warm-up steps, while the clock ramps from idle
DIST_S = 1.0  # the per-call timing window after the timed region (clock sampled there)
MIN_CLOCK_SAMPLES = 10


def kernel_source_digest(key: str) -> str:
    """sha256 of the kernel's sources with comments and blank space removed,
    so that only a change to the code itself invalidates stored counters."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES[key]:
        with open(os.path.join(_CSRC, name)) as f:
            text = f.read()
        text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
        text = re.sub(r"//[^\n]*", " ", text)
        h.update(" ".join(text.split()).encode())
    return h.hexdigest()


def workload_by_name(name: str):
    """(workload, kernel key) for a square or a key/value-cache workload."""
    from io_aware_tiled_08_amd import workloads as W
    if name in W.WORKLOADS:
        w = W.WORKLOADS[name]
        return w, w.dtype
    if name in W.CACHE_WORKLOADS:
        return W.CACHE_WORKLOADS[name], "kvcache"
    if name in W.FP8_WORKLOADS:
        return W.FP8_WORKLOADS[name], "fp8"
    if name in W.BWD_WORKLOADS:
        return W.BWD_WORKLOADS[name], "bwd"
    raise SystemExit(f"unknown workload {name!r}; known: "
                     f"{sorted(W.WORKLOADS) + sorted(W.CACHE_WORKLOADS) + sorted(W.FP8_WORKLOADS)}"
                     f" + {sorted(W.BWD_WORKLOADS)}")


def traffic_path(workload: str) -> str:
    return os.path.join(PROFILES, f"traffic_{workload}.md")


def measured_traffic(workload: str, key: str):
    """HBM bytes per launch from the committed counter summary, or None when
    there is none or the kernel source changed since it was taken."""
    path = traffic_path(workload)
    if not os.path.exists(path):
        return None
    text = open(path).read()
    sha = re.search(r"^kernel_source_sha256:\s*([0-9a-f]{64})\s*$", text, re.M)
    val = re.search(r"^hbm_bytes_per_launch:\s*([0-9.eE+]+)\s*$", text, re.M)
    if not sha or not val or sha.group(1) != kernel_source_digest(key):
        return None
    return float(val.group(1))


def host_cpu():
    """(cores this process may use, CPU model name)."""
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:  # non-Linux
        cores = os.cpu_count() or 1
    model = ""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    model = line.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return cores, model


def run_oracle_pool(units, run_unit, budget_s: float):
    """Runs run_unit(u) for the units in order on a pool of threads, one per
    core (at most 16), each with one BLAS thread: numpy releases the
    interpreter lock inside its array loops and BLAS products, so the units
    run in parallel.  New units are started until budget_s has passed (at
    least one).  Returns (sum of what the finished units returned, their
    count, elapsed seconds, threads)."""
    from concurrent.futures import FIRST_COMPLETED, ThreadPoolExecutor, wait

    from threadpoolctl import threadpool_limits
    cores, _ = host_cpu()
    workers = max(1, min(cores, 16))
    total, count = 0.0, 0
    it = iter(units)
    t0 = time.perf_counter()
    with threadpool_limits(1), ThreadPoolExecutor(workers) as ex:
        pending, exhausted = set(), False
        while True:
            while (not exhausted and len(pending) < 2 * workers
                   and (count + len(pending) == 0 or time.perf_counter() - t0 < budget_s)):
                u = next(it, None)
                if u is None:
                    exhausted = True
                    break
                pending.add(ex.submit(run_unit, u))
            if not pending:
                break
            done, pending = wait(pending, return_when=FIRST_COMPLETED)
            for f in done:
                total += f.result()
                count += 1
    return total, count, time.perf_counter() - t0, workers


def _baseline_record(value, unit, workers, sample):
    cores, model = host_cpu()
    return {"value": value, "unit": unit, "cores": workers, "kind": "oracle", "sample": sample,
            "host_cores": cores, "cpu_model": model}


def cpu_baseline(w, q, k, v, budget_s: float, gpu_out=None):
    """Times the fp64 oracle on the workload's own inputs in blocks of 512
    query rows (heads in order, rows in order) on a thread pool over the host's
    cores, starting blocks until the budget is spent.  FLOPs are counted per
    row from the number of keys the row sees (4*d per visible key).  With
    gpu_out = (O, LSE), the GPU's outputs on the host, the record also gives
    the largest absolute difference of O and of LSE from the oracle over the
    rows the oracle computed."""
    import threading

    import numpy as np

    import oracle
    block = 512
    units = [(b, h, r0) for b in range(w.B) for h in range(w.H) for r0 in range(0, w.N, block)]
    err = {"O": 0.0, "LSE": 0.0}
    lock = threading.Lock()

    def run(u):
        b, h, r0 = u
        sl = (slice(b, b + 1), slice(h, h + 1))
        idx = np.arange(r0, min(r0 + block, w.N), dtype=np.int64)
        O_ref, L_ref = oracle.attention_forward(q[sl], k[sl], v[sl], w.scale, w.causal, rows=idx)
        if gpu_out is not None:
            eo = float(np.max(np.abs(gpu_out[0][b, h, idx].astype(np.float64) - O_ref[0, 0])))
            el_ = float(np.max(np.abs(gpu_out[1][b, h, idx].astype(np.float64) - L_ref[0, 0])))
            with lock:
                err["O"] = max(err["O"], eo)
                err["LSE"] = max(err["LSE"], el_)
        visible = (idx + 1) if w.causal else np.full(idx.shape, w.N)
        return 4.0 * w.d * float(visible.sum())

    flops, n, el, workers = run_oracle_pool(units, run, budget_s)
    rows_done = sum(min(block, w.N - units[i][2]) for i in range(n))
    rec = _baseline_record(
        flops / el / 1e12, "TFLOP/s", workers,
        f"{rows_done} of {w.B * w.H * w.N} query rows of {w.name} (the first {n} blocks of "
        f"{block} rows, heads in order), fp64 numpy, {workers} threads, {el:.1f} s")
    rec["seconds"] = round(el, 2)
    rec["rows"] = rows_done
    if gpu_out is not None:
        rec["max_abs_err"] = {"O": err["O"], "LSE": err["LSE"], "rows": rows_done}
    return rec


def _counter_rows(path, counter):
    rows = []
    with open(path) as f:
        for r in csv.DictReader(f):
            if r["Counter_Name"] == counter:
                rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def summarize_traffic(fetch_csv: str, write_csv: str, workload: str) -> str:
    """Turns two rocprofv3 --pmc runs (FETCH_SIZE, WRITE_SIZE; KiB per
    dispatch) of `bench.py --copy-calibration` into HBM bytes per launch of
    the attention kernel, scaled by what the same counters read for the
    calibration copies, and writes profiles/traffic_<workload>.md."""
    w, key = workload_by_name(workload)
    main_pat, all_pat = KERNEL_NAME_PATTERN[key]
    out = {}
    for counter, path in (("FETCH_SIZE", fetch_csv), ("WRITE_SIZE", write_csv)):
        rows = _counter_rows(path, counter)
        calls = [v for n, v in rows if main_pat in n]
        fa = [v for n, v in rows if all_pat in n]
        cp = [v for n, v in rows if "copy" in n.lower() or "elementwise" in n.lower()]
        cp = [v for v in cp if v > 0.5 * COPY_BYTES / 1024]  # the 512 MiB copies only
        if not calls or not cp:
            raise SystemExit(f"{path}: no {counter} rows for the kernel ({len(calls)}) or the copy ({len(cp)})")
        copy_kib = sum(cp) / len(cp)
        factor = (COPY_BYTES / 1024) / copy_kib
        fa_kib = sum(fa) / len(calls)  # every kernel of one call, per call
        out[counter] = {"kernel_kib": fa_kib, "copy_kib": copy_kib, "factor": factor,
                        "bytes": fa_kib * 1024 * factor, "n": len(calls)}
    total = out["FETCH_SIZE"]["bytes"] + out["WRITE_SIZE"]["bytes"]
    comp = w.compulsory_bytes()
    os.makedirs(PROFILES, exist_ok=True)
    lines = [
        f"# HBM traffic of the attention kernels, workload {workload}",
        "",
        f"Workload: {w.description}.  Compulsory bytes (every input read once, every output",
        f"written once): {comp} ({comp / 2**20:.2f} MiB).  Kernels counted per call: "
        f"`{all_pat}*` (dispatches of `{main_pat}` = calls).",
        "",
        "Commands (GPU host, from the repository root):",
        "",
        "    rocprofv3 --pmc FETCH_SIZE -f csv -d gpurun_out/traffic_" + workload + "/fetch -o fetch -- \\",
        f"        python3 bench.py --workload {workload} --steps 5 --warmup 1 --settle 0 --dist 0 "
        "--cpu-budget 0 --copy-calibration",
        "    rocprofv3 --pmc WRITE_SIZE -f csv -d gpurun_out/traffic_" + workload + "/write -o write -- \\",
        f"        python3 bench.py --workload {workload} --steps 5 --warmup 1 --settle 0 --dist 0 "
        "--cpu-budget 0 --copy-calibration",
        "    python3 bench.py --workload " + workload + " --summarize-traffic \\",
        "        gpurun_out/traffic_" + workload + "/fetch/fetch_counter_collection.csv \\",
        "        gpurun_out/traffic_" + workload + "/write/write_counter_collection.csv",
        "",
        "| counter | kernel KiB/call (mean) | calls | 512 MiB copy reads as KiB | scale factor | bytes/call |",
        "|---|---|---|---|---|---|",
    ]
    for counter in ("FETCH_SIZE", "WRITE_SIZE"):
        o = out[counter]
        lines.append(f"| {counter} | {o['kernel_kib']:.1f} | {o['n']} | {o['copy_kib']:.1f} | "
                     f"{o['factor']:.4f} | {o['bytes']:.0f} |")
    lines += [
        "",
        f"HBM bytes per launch (fetch + write, calibrated): {total:.0f} "
        f"({total / comp:.3f} x compulsory).",
        "",
        "Machine-readable (bench.py reads these; traffic is reported only while the",
        "kernel source hash matches):",
        "",
        f"hbm_bytes_per_launch: {total:.0f}",
        f"kernel_source_sha256: {kernel_source_digest(key)}",
        "",
    ]
    path = traffic_path(workload)
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


SQ_PASSES = (
    "SQ_INSTS_VALU SQ_INSTS_MFMA SQ_INSTS_LDS SQ_INSTS_SALU SQ_ACTIVE_INST_VALU SQ_ACTIVE_INST_LDS "
    "SQ_WAIT_ANY SQ_WAIT_INST_ANY GRBM_GUI_ACTIVE",
    "SQ_INST_LEVEL_LDS SQ_INSTS_LDS_LOAD_BANDWIDTH SQ_LDS_IDX_ACTIVE SQ_BUSY_CYCLES SQ_ACTIVE_INST_ANY "
    "SQ_ACTIVE_INST_SCA SQ_VALU_MFMA_BUSY_CYCLES SQ_WAVE_CYCLES GRBM_GUI_ACTIVE",
    "SQ_VALU_MFMA_COEXEC_CYCLES SQ_WAIT_INST_LDS SQ_INSTS_VALU_TRANS_F32 SQ_INSTS_VALU_CVT SQ_INSTS_SMEM "
    "SQ_INSTS_VMEM SQ_LDS_ADDR_CONFLICT SQ_LDS_UNALIGNED_STALL GRBM_GUI_ACTIVE",
)
N_XCD, N_CU, N_SIMD = 8, 256, 1024


SQ_UNITS = (
    "GRBM_GUI_ACTIVE is summed over the 8 XCDs, so one XCD's busy cycles are GRBM_GUI_ACTIVE / 8 "
    "(in a counter run that also holds the dispatch's own set-up, so fractions over it are lower "
    "bounds).  SQ_WAVE_CYCLES, SQ_WAIT_* and SQ_ACTIVE_INST_* count quad-cycles (4 cycles); "
    "SQ_VALU_MFMA_BUSY_CYCLES and SQ_VALU_MFMA_COEXEC_CYCLES count cycles per SIMD, summed over the "
    "1024 SIMDs; SQ_INSTS_VALU includes the MFMA instructions; SQ_INSTS_LDS_LOAD_BANDWIDTH counts "
    "64-byte units.")


def summarize_counters(csvs, workload: str) -> str:
    """Turns the three SQ counter passes (rocprofv3 --pmc with the counter
    sets of SQ_PASSES, one run of bench.py each) into
    profiles/sq_counters_<workload>.md: per kernel of the workload, the mean
    of each counter per dispatch and the ratios read from them (units as
    SQ_UNITS states)."""
    w, key = workload_by_name(workload)
    _, all_pat = KERNEL_NAME_PATTERN[key]
    vals = {}
    for path in csvs:
        with open(path) as f:
            for r in csv.DictReader(f):
                if all_pat in r["Kernel_Name"]:
                    vals.setdefault(r["Kernel_Name"], {}).setdefault(r["Counter_Name"], []).append(
                        float(r["Counter_Value"]))
    if not vals:
        raise SystemExit(f"no dispatches of {all_pat}* in {csvs}")
    lines = [
        f"# SQ counters, workload {workload}",
        "",
        f"Workload: {w.description}.",
        "",
        "Commands (GPU host; R = the repository root; rocprofv3 run from /tmp with TMPDIR=/tmp),",
        "one run per counter set, at most 8 SQ counters each:",
        "",
    ]
    for i, counters in enumerate(SQ_PASSES, 1):
        lines += [f"    rocprofv3 --pmc {counters} \\",
                  f"        -f csv -d $R/gpurun_out/sq_{workload}/p{i} -o p -- python3 $R/bench.py --workload {workload} "
                  "--steps 5 --warmup 2 --settle 0 --dist 0 --cpu-budget 0"]
    lines += [f"    python3 bench.py --workload {workload} --summarize-counters "
              + " ".join(f"gpurun_out/sq_{workload}/p{i}/p_counter_collection.csv" for i in (1, 2, 3)),
              "", "Units: " + SQ_UNITS, ""]
    for name, c in sorted(vals.items()):
        m = {k: sum(v) / len(v) for k, v in c.items()}
        lines += [f"## `{name[:110]}`", "", "| counter | mean per dispatch | dispatches |", "|---|---|---|"]
        lines += [f"| {k} | {m[k]:.4g} | {len(c[k])} |" for k in sorted(m)]
        g = lambda k: m.get(k)  # noqa: E731
        derived = []
        if g("GRBM_GUI_ACTIVE"):
            length = g("GRBM_GUI_ACTIVE") / N_XCD
            derived.append(f"busy length (GRBM_GUI_ACTIVE / {N_XCD}): {length:.0f} cycles")
            if g("SQ_VALU_MFMA_BUSY_CYCLES") is not None:
                derived.append("matrix pipe busy per SIMD over that length: "
                               f"{g('SQ_VALU_MFMA_BUSY_CYCLES') / (length * N_SIMD):.1%}")
        if g("SQ_VALU_MFMA_COEXEC_CYCLES") is not None and g("SQ_VALU_MFMA_BUSY_CYCLES"):
            derived.append("vector instructions issued while the matrix pipe is busy / matrix busy: "
                           f"{g('SQ_VALU_MFMA_COEXEC_CYCLES') / g('SQ_VALU_MFMA_BUSY_CYCLES'):.1%}")
        wave = g("SQ_WAVE_CYCLES")
        if wave:
            for k, label in (("SQ_WAIT_ANY", "wave time at a wait-count instruction"),
                             ("SQ_WAIT_INST_ANY", "wave time with an instruction ready but not issued"),
                             ("SQ_WAIT_INST_LDS", "wave time waiting to issue an LDS instruction")):
                if g(k) is not None:
                    derived.append(f"{label} ({k} / SQ_WAVE_CYCLES): {g(k) / wave:.1%}")
        if g("SQ_ACTIVE_INST_VALU") and g("SQ_INSTS_VALU"):
            derived.append("cycles per vector instruction (4 x SQ_ACTIVE_INST_VALU / SQ_INSTS_VALU): "
                           f"{4 * g('SQ_ACTIVE_INST_VALU') / g('SQ_INSTS_VALU'):.2f}")
        if g("SQ_INSTS_LDS_LOAD_BANDWIDTH") is not None and g("SQ_LDS_IDX_ACTIVE"):
            b = 64 * g("SQ_INSTS_LDS_LOAD_BANDWIDTH")
            derived.append(f"LDS bytes read: {b:.4g}; per LDS-active cycle and CU: "
                           f"{b / g('SQ_LDS_IDX_ACTIVE'):.0f}")
        if key in ("f16", "bf16") and not w.causal and "fwd_f16_" in name and g("SQ_INSTS_MFMA"):
            # one wave-tile = 32 query rows of one wave against one 128-key tile
            n_wt = w.B * w.H * ((w.N + 31) // 32) * ((w.N + 127) // 128)
            per = ", ".join(f"{label} {x / n_wt:.1f}" for label, x in (
                ("vector (not MFMA)", g("SQ_INSTS_VALU") - g("SQ_INSTS_MFMA")),
                ("MFMA", g("SQ_INSTS_MFMA")), ("of them exp", g("SQ_INSTS_VALU_TRANS_F32")),
                ("conversions", g("SQ_INSTS_VALU_CVT")), ("LDS", g("SQ_INSTS_LDS")),
                ("scalar", g("SQ_INSTS_SALU")), ("vector memory", g("SQ_INSTS_VMEM")))
                if x is not None)
            derived.append(f"instructions per wave-tile (32 rows x 128 keys, {n_wt} per dispatch): {per}")
        lines += ["", "Read from them:", ""] + [f"- {x}" for x in derived] + [""]
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"sq_counters_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


def summarize_trace(trace_dir: str, bench_log: str, workload: str) -> str:
    """Turns one `rocprofv3 --kernel-trace --stats -f csv` run of bench.py
    (its output directory and the run's stdout) into
    profiles/kernel_trace_<workload>.md: the stats table and, per kernel, the
    average duration of the dispatches that fell in the timed region (the
    calls after the clock settling and the warm-up steps, as the JSON line
    reports them), next to the same run's event timing."""
    w, key = workload_by_name(workload)
    main_pat, all_pat = KERNEL_NAME_PATTERN[key]

    def find(suffix):
        for dirpath, _, files in os.walk(trace_dir):
            for f in files:
                if f.endswith(suffix):
                    return os.path.join(dirpath, f)
        raise SystemExit(f"{trace_dir}: no *{suffix}")

    stats = [r for r in csv.DictReader(open(find("kernel_stats.csv"))) if all_pat in r["Name"]]
    trace = [r for r in csv.DictReader(open(find("kernel_trace.csv"))) if all_pat in r["Kernel_Name"]]
    r = json.loads([line for line in open(bench_log) if line.startswith("{")][-1])
    rf = r["roofline"]
    graph = r.get("launch") == "hip_graph"
    # settle calls, warm-up steps and, with --graph, the untimed replay
    first = r.get("clock_settle", {}).get("calls", 0) + r["warmup"] + (r["steps"] if graph else 0)
    by = {}
    for t in trace:
        by.setdefault(t["Kernel_Name"], []).append(
            (int(t["Start_Timestamp"]), int(t["End_Timestamp"]) - int(t["Start_Timestamp"])))
    parts, total = [], 0.0
    for name, v in by.items():
        v.sort()
        timed = [d for _, d in v[first:first + r["steps"]]]
        avg = sum(timed) / len(timed)
        total += avg
        parts.append(f"`{name[:70]}` {avg:.0f} ns over {len(timed)} dispatches")
    ev_ns = rf["kernel_ms"] * 1e6
    cmd = " ".join(a for a in ["python3 bench.py --workload", workload, "--steps", str(r["steps"]),
                               "--cpu-budget 0"] + (["--graph"] if graph else []))
    lines = [
        f"# Kernel trace, workload {workload}",
        "",
        f"Workload: {w.description}.",
        "",
        "Command (GPU host, repository root; then `bench.py --summarize-trace`):",
        "",
        f"    rocprofv3 --kernel-trace --stats -f csv -d gpurun_out/prof/trace_{workload} -o trace -- \\",
        f"        {cmd} > gpurun_out/prof/bench_{workload}.log",
        f"    python3 bench.py --workload {workload} --summarize-trace gpurun_out/prof/trace_{workload} "
        f"gpurun_out/prof/bench_{workload}.log",
        "",
        "Stats over every dispatch of the run (clock settling, warm-up, timed and per-call timed calls; ns):",
        "",
        "| kernel | calls | average ns | min ns | max ns | stddev ns |",
        "|---|---|---|---|---|---|",
    ]
    for st in stats:
        lines.append(f"| `{st['Name']}` | {st['Calls']} | {float(st['AverageNs']):.0f} | "
                     f"{float(st['MinNs']):.0f} | {float(st['MaxNs']):.0f} | {float(st['StdDev']):.0f} |")
    lines += [
        "",
        "Timed region (dispatches " + f"{first} .. {first + r['steps'] - 1} of each kernel): "
        + "; ".join(parts) + ".",
        "",
        f"Same run, HIP events on the launch stream around the {r['steps']} timed calls"
        f"{' (one replay of a captured HIP graph)' if graph else ''}: {ev_ns:.0f} ns per call, "
        f"{r['value']} {r['unit']} ({100 * rf['frac']:.1f}% of {rf['peak']} {rf['unit']}); graphics clock "
        f"median {rf.get('gfx_clock_mhz_median')} MHz, socket power median "
        f"{rf.get('socket_power_w_median')} W (per-call window after the timed region).  Trace average "
        f"(sum over the call's kernels) / event average = {total / ev_ns:.3f}.",
        "",
    ]
    os.makedirs(PROFILES, exist_ok=True)
    path = os.path.join(PROFILES, f"kernel_trace_{workload}.md")
    with open(path, "w") as f:
        f.write("\n".join(lines))
    return path


def percentile(sorted_vals, f):
    """Nearest-rank percentile of an ascending list."""
    i = min(len(sorted_vals) - 1, max(0, int(round(f * (len(sorted_vals) - 1)))))
    return sorted_vals[i]


class ClockSampler:
    """Samples the GPU's graphics clock (MHz) through amdsmi in a background
    thread, with the time of each sample.  Reading the clock changes no
    setting; when amdsmi is missing or refuses, no samples are taken and the
    clock fields are left out."""

    def __init__(self, period_s=0.01):
        self.period_s = period_s
        self.samples = []
        self.power = []
        self._stop = None
        self._thread = None

    def _power(self, amdsmi, h):
        """Socket power in watts, or None."""
        try:
            info = amdsmi.amdsmi_get_power_info(h)
        except Exception:
            return None
        for key in ("current_socket_power", "socket_power", "average_socket_power"):
            x = info.get(key) if isinstance(info, dict) else None
            if isinstance(x, (int, float)) and 0 < x < 5000:
                return float(x)
        return None

    def _read(self, amdsmi, h):
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            vals = m.get("current_gfxclks")
            if isinstance(vals, (list, tuple)):
                vals = [x for x in vals if isinstance(x, (int, float)) and 0 < x < 10000]
                if vals:
                    return sum(vals) / len(vals)
            x = m.get("current_gfxclk")
            if isinstance(x, (int, float)) and 0 < x < 10000:
                return float(x)
        except Exception:
            pass
        info = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.GFX)
        x = info.get("clk")
        return float(x) if isinstance(x, (int, float)) and 0 < x < 10000 else None

    def start(self):
        import threading
        try:
            import amdsmi
            amdsmi.amdsmi_init()
            handles = amdsmi.amdsmi_get_processor_handles()
            if not handles:
                return
            h = handles[0]
        except Exception:
            return
        self._stop = threading.Event()

        def run():
            while not self._stop.is_set():
                try:
                    x = self._read(amdsmi, h)
                except Exception:
                    return
                if x:
                    self.samples.append((time.perf_counter(), x))
                w = self._power(amdsmi, h)
                if w:
                    self.power.append((time.perf_counter(), w))
                self._stop.wait(self.period_s)

        self._thread = threading.Thread(target=run, daemon=True)
        self._thread.start()

    def stop(self):
        if self._thread is not None:
            self._stop.set()
            self._thread.join(timeout=2.0)
        try:
            import amdsmi
            amdsmi.amdsmi_shut_down()
        except Exception:
            pass

    def window(self, t0, t1, power=False):
        """Clock (or power) samples taken between perf_counter times t0 and t1."""
        return [x for t, x in (self.power if power else self.samples) if t0 <= t <= t1]


def calibrate(seconds: float = 1.5) -> None:
    """Reachable fp16 matrix throughput on this card, with the clock and socket
    power held under it: hipBLASLt square GEMMs (torch.matmul, n = 8192 and
    16384) and register-only chains of f16 MFMAs (libfa_calib.so, 256
    workgroups x 8 waves, 131072 FLOPs per wave and step) for the 32x32x16 and
    16x16x32 shapes, each with small and with unit-variance operands.  Prints
    one JSON line per case.  The
    attention kernel's roofline fraction is quoted against the published dense
    peak; these lines say how much of that peak the card sustains at all
    under its power limit."""
    import ctypes

    import torch

    from io_aware_tiled_08_amd.build import CALIB_LIB_PATH, build_calibration_library
    if not os.path.exists(CALIB_LIB_PATH):
        build_calibration_library()
    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)

    def measure(label, fn, reps, flops):
        t = time.perf_counter()
        while time.perf_counter() - t < seconds:  # clock settling
            for _ in range(3):
                fn()
            torch.cuda.synchronize()
        clk = ClockSampler()
        clk.start()
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        t0 = time.perf_counter()
        s.record(stream)
        for _ in range(reps):
            fn()
        e.record(stream)
        torch.cuda.synchronize()
        t1 = time.perf_counter()
        clk.stop()
        ms = s.elapsed_time(e) / reps
        tf = flops / (ms * 1e-3) / 1e12
        mhz = sorted(clk.window(t0, t1))
        watts = sorted(clk.window(t0, t1, power=True))
        print(json.dumps({"calibration": label, "ms": round(ms, 4), "tflops": round(tf, 1),
                          "frac_of_peak": round(tf / MFMA_PEAK_TFLOPS["f16"], 4),
                          "clock_mhz_median": percentile(mhz, 0.5) if mhz else None,
                          "socket_power_w_median": percentile(watts, 0.5) if watts else None,
                          "samples": len(mhz), "window_s": round(t1 - t0, 3)}), flush=True)

    for n, reps in ((8192, 400), (16384, 50)):
        a = torch.randn(n, n, device=dev, dtype=torch.float16)
        b = torch.randn(n, n, device=dev, dtype=torch.float16)
        c = torch.empty(n, n, device=dev, dtype=torch.float16)
        measure(f"gemm_f16_n{n}", lambda: torch.matmul(a, b, out=c), reps, 2.0 * n ** 3)
        del a, b, c
    lib = ctypes.CDLL(CALIB_LIB_PATH)
    lib.fa_calib_mfma.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                                  ctypes.c_void_p]
    blocks, iters = 256, 20000
    out = torch.empty(blocks * 512, device=dev)
    for shape, label in enumerate(("32x32x16", "16x16x32", "32x32x16_unitvar",
                                   "16x16x32_unitvar")):
        def chain(shape=shape):
            rc = lib.fa_calib_mfma(out.data_ptr(), blocks, iters, shape, stream.cuda_stream)
            if rc != 0:
                raise RuntimeError(f"fa_calib_mfma failed ({rc})")
        measure(f"mfma_chain_f16_{label}", chain, 20, float(blocks) * 8 * iters * 131072)


# The configurations of the forward path side by side (bench.py --all-configs):
# (label, workload, extra bench.py arguments).  The single-head fp32 kernel is
# shorter than a launch from Python, so its steps run as one captured graph.
ALL_CONFIGS = (
    ("C1", "single_head_f32", ("--graph",)),
    ("C2 non-causal", "batch_f16_d64", ()),
    ("C2 causal", "batch_f16_d64_causal", ()),
    ("C3 (headline)", "headline_f16_d128", ()),
    ("C4", "rescale_stress_bf16", ()),
    ("C5", "long_context_bf16", ()),
)


def all_configs(steps: int, budget_s: float, out_path: str) -> str:
    """Runs bench.py once per configuration of ALL_CONFIGS, each in a child
    process, and writes one table of them to out_path: GPU rate and share of
    the MFMA peak, HBM GB/s of compulsory and of counter-measured bytes (the
    committed traffic profile, when the kernel source matches), the largest
    difference of O and LSE from the fp64 oracle over the rows the CPU
    baseline computed, and that baseline's time and threads."""
    import subprocess
    recs = []
    for label, wl, extra in ALL_CONFIGS:
        cmd = [sys.executable, os.path.abspath(__file__), "--workload", wl, "--steps", str(steps),
               "--cpu-budget", str(budget_s), *extra]
        print(f"step: {label} ({wl})", flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True,
                           timeout=600)
        if r.returncode != 0:
            raise SystemExit(f"{wl} failed ({r.returncode}):\n{r.stderr[-2000:]}")
        line = [x for x in r.stdout.splitlines() if x.startswith("{")][-1]
        print(line, flush=True)
        recs.append((label, json.loads(line)))
    text = format_all_configs(recs, steps, budget_s)
    with open(out_path, "w") as f:
        f.write(text)
    return text


def format_all_configs(recs, steps: int, budget_s: float) -> str:
    """The markdown table of all_configs from (label, bench JSON record) pairs."""
    cmdline = (f"python3 bench.py --all-configs --steps {steps} --cpu-budget {budget_s:g}")
    out = ["# All forward configurations side by side", "",
           "Command (GPU host, repository root; one bench.py child process per configuration):", "",
           f"    {cmdline}", "",
           "GB/s columns are bytes per launch over the event-timed kernel time: compulsory bytes "
           "(every input read once, every output written once) and counter-measured HBM bytes "
           "(`profiles/traffic_<workload>.md`, FETCH_SIZE + WRITE_SIZE calibrated against a "
           "copy of known size), as fractions of 8 TB/s.  Errors are max |GPU - oracle| over the "
           "rows the CPU baseline computed (fp64 oracle on the same inputs).", "",
           "| config | workload | GPU TFLOP/s | % of MFMA peak | compulsory GB/s (of 8 TB/s) | "
           "counter GB/s (of 8 TB/s) | max abs err O / LSE (rows) | oracle CPU s (threads) |",
           "|---|---|---|---|---|---|---|---|"]
    for label, r in recs:
        rf = r["roofline"]
        ms = rf["kernel_ms"]
        comp = rf["compulsory_bytes"] / (ms * 1e-3) / 1e9
        cnt = rf.get("traffic")
        cnt_s = (f"{cnt / (ms * 1e-3) / 1e9:.0f} ({cnt / (ms * 1e-3) / 8e12:.1%})"
                 if cnt else "n/a")
        cb = r.get("cpu_baseline") or {}
        err = cb.get("max_abs_err")
        err_s = (f"{err['O']:.2e} / {err['LSE']:.2e} ({err['rows']})" if err else "n/a")
        cpu_s = (f"{cb.get('seconds', float('nan')):.1f} ({cb.get('cores')})" if cb else "n/a")
        out.append(f"| {label} | `{r['config']['workload']}` | {r['value']:.1f} | {rf['frac']:.1%} | "
                   f"{comp:.0f} ({comp / 8000:.1%}) | {cnt_s} | {err_s} | {cpu_s} |")
    return "\n".join(out) + "\n"


def cpu_baseline_cache(w, q, k, v, budget_s: float):
    """Times the fp64 oracle on a key/value-cache workload, whole (b, h) heads
    on a thread pool over the host's cores until the budget is spent; the rate
    is the compulsory bytes of the heads done per second, like the GPU figure."""
    import oracle
    per_head = w.compulsory_bytes() / (w.B * w.H)

    def run(u):
        b, h = u
        sl = (slice(b, b + 1), slice(h, h + 1))
        oracle.attention_forward(q[sl], k[sl], v[sl], w.scale, w.causal)
        return per_head

    done_bytes, heads, el, workers = run_oracle_pool(
        [(b, h) for b in range(w.B) for h in range(w.H)], run, budget_s)
    return _baseline_record(
        done_bytes / el / 1e9, "GB/s", workers,
        f"{heads} of {w.B * w.H} (b,h) heads of {w.name}, all {w.Nq} query rows each, "
        f"fp64 numpy, {workers} threads, {el:.1f} s")


def cpu_baseline_bwd(w, q, k, v, do, budget_s: float):
    """Times the fp64 backward oracle, whole (b, h) heads on a thread pool
    over the host's cores until the budget is spent; FLOPs as the workload
    counts them."""
    import oracle
    per_head = w.flops() / (w.B * w.H)

    def run(u):
        b, h = u
        sl = (slice(b, b + 1), slice(h, h + 1))
        oracle.attention_backward(q[sl], k[sl], v[sl], do[sl], w.scale, w.causal)
        return per_head

    flops, heads, el, workers = run_oracle_pool(
        [(b, h) for b in range(w.B) for h in range(w.H)], run, budget_s)
    return _baseline_record(
        flops / el / 1e12, "TFLOP/s", workers,
        f"{heads} of {w.B * w.H} (b,h) heads of {w.name}, whole heads, fp64 numpy, "
        f"{workers} threads, {el:.1f} s")


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=None,
                    help="untimed warm-up steps (default 10), after 1.5 s of untimed calls that "
                         "let the GPU clock reach its loaded steady state")
    ap.add_argument("--settle", type=float, default=SETTLE_S,
                    help="seconds of untimed calls before the warm-up steps (clock settling)")
    ap.add_argument("--dist", type=float, default=DIST_S,
                    help="seconds of per-call timing after the timed region (the clock and power "
                         "are read there; 0 = 20 calls)")
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time for cpu_baseline (0 = skip)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="after the timed region, run device copies of a known size "
                         "(for calibrating rocprofv3 FETCH_SIZE / WRITE_SIZE)")
    ap.add_argument("--persistent", type=int, default=None, metavar="NWG",
                    help="run an fp16/bf16 forward workload on the persistent schedule with NWG "
                         "resident workgroups (0 = one per CU)")
    ap.add_argument("--graph", action="store_true",
                    help="time the steps as one captured HIP graph (square forward workloads): "
                         "removes host launch gaps for kernels shorter than a launch")
    ap.add_argument("--all-configs", action="store_true",
                    help="run every forward configuration (C1-C5) in child processes and write "
                         "profiles/all_configs.md")
    ap.add_argument("--calibrate", action="store_true",
                    help="print the card's sustained fp16 GEMM and register-only MFMA throughput "
                         "with clock and power, then exit")
    ap.add_argument("--summarize-traffic", nargs=2, metavar=("FETCH_CSV", "WRITE_CSV"),
                    help="write profiles/traffic_<workload>.md from two rocprofv3 --pmc runs")
    ap.add_argument("--summarize-counters", nargs=3, metavar=("P1_CSV", "P2_CSV", "P3_CSV"),
                    help="write profiles/sq_counters_<workload>.md from the three SQ counter passes")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "BENCH_LOG"),
                    help="write profiles/kernel_trace_<workload>.md from a rocprofv3 --kernel-trace "
                         "--stats run of bench.py and that run's output")
    args = ap.parse_args()

    from io_aware_tiled_08_amd import workloads as W
    name = args.workload or W.HEADLINE
    if args.summarize_traffic:
        print(summarize_traffic(*args.summarize_traffic, name))
        return
    if args.summarize_trace:
        print(summarize_trace(*args.summarize_trace, name))
        return
    if args.summarize_counters:
        print(summarize_counters(args.summarize_counters, name))
        return
    if args.calibrate:
        calibrate()
        return
    if args.all_configs:
        print(all_configs(args.steps, args.cpu_budget,
                          os.path.join(os.path.dirname(os.path.abspath(__file__)), "profiles",
                                       "all_configs.md")))
        return
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the forward pass "
              "shards by (batch, head) with no communication, and this build measures "
              "one GPU's share.", file=sys.stderr)
        sys.exit(2)
    w, key = workload_by_name(name)
    cache = key == "kvcache"
    if args.persistent is not None and key not in ("f16", "bf16"):
        raise SystemExit("--persistent applies to the fp16/bf16 forward workloads")
    if args.graph and key not in ("f16", "bf16", "f32"):
        raise SystemExit("--graph applies to the square forward workloads")

    import torch

    from io_aware_tiled_08_amd import binding, flash_attn_fwd, flash_attn_fwd_kvcache
    if not os.path.exists(binding.library_path()):
        from io_aware_tiled_08_amd.build import build_library
        build_library()

    dev = torch.device("cuda:0")
    stream = torch.cuda.current_stream(dev)
    if cache:
        q, k, v = W.cache_workload_inputs(w)
        qd, kd, vd = (x.to(dev) for x in (q, k, v))
        o = torch.empty_like(qd)
        lse = torch.empty((w.B, w.H, w.Nq), dtype=torch.float32, device=dev)
        n_split = binding.kvcache_splits(w.B, w.H, w.Nq, w.Nk, w.d, 0)
        ws_bytes = binding.kvcache_workspace_size(w.B, w.H, w.Nq, w.Nk, w.d, 0)
        ws = torch.empty(max(ws_bytes, 16), dtype=torch.uint8, device=dev)

        def step():
            flash_attn_fwd_kvcache(qd, kd, vd, o, lse, scale=w.scale, causal=w.causal,
                                   workspace=ws, stream=stream)
    elif key == "bwd":
        from io_aware_tiled_08_amd import flash_attn_bwd
        q, k, v = W.random_qkv(w.B, w.H, w.N, w.d, w.dtype, w.seed)
        do = W.random_dout(w.B, w.H, w.N, w.d, w.dtype, w.seed)
        qd, kd, vd, dod = (x.to(dev) for x in (q, k, v, do))
        o, lse = flash_attn_fwd(qd, kd, vd, scale=w.scale, causal=w.causal)
        dq, dk, dv = (torch.empty_like(qd) for _ in range(3))
        ws = torch.empty(max(binding.lib().flash_attn_bwd_workspace_size(w.B, w.H, w.N), 16),
                         dtype=torch.uint8, device=dev)

        def step():
            flash_attn_bwd(qd, kd, vd, o, lse, dod, dq, dk, dv, scale=w.scale, causal=w.causal,
                           workspace=ws, stream=stream)
    elif key == "fp8":
        from io_aware_tiled_08_amd import flash_attn_fwd_fp8
        q, k, v, qs, ks, vs = W.fp8_workload_inputs(w)
        qd, kd, vd = (x.to(dev) for x in (q, k, v))
        o = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=dev)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def step():
            flash_attn_fwd_fp8(qd, kd, vd, o, lse, q_descale=qs, k_descale=ks, v_descale=vs,
                               scale=w.scale, causal=w.causal, stream=stream)
    elif args.persistent is not None:
        from io_aware_tiled_08_amd import flash_attn_fwd_persistent
        q, k, v = W.workload_inputs(w)
        qd, kd, vd = (x.to(dev) for x in (q, k, v))
        o = torch.empty_like(qd)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def step():
            flash_attn_fwd_persistent(qd, kd, vd, o, lse, scale=w.scale, causal=w.causal,
                                      num_workgroups=args.persistent, stream=stream)
    else:
        q, k, v = W.workload_inputs(w)
        qd, kd, vd = (x.to(dev) for x in (q, k, v))
        o = torch.empty_like(qd)
        lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)

        def step():
            flash_attn_fwd(qd, kd, vd, o, lse, scale=w.scale, causal=w.causal, stream=stream)

    clock = ClockSampler()
    clock.start()
    # Clock settling, before the warm-up steps: the card starts from its idle
    # clock and takes about a second of sustained load to reach the clock it
    # holds under this kernel (power-limited, below the 2.4 GHz peak).  These
    # calls are untimed and reported in the JSON line as "clock_settle".
    settle_calls = 0
    t_s = time.perf_counter()
    while time.perf_counter() - t_s < args.settle:
        for _ in range(10):
            step()
        settle_calls += 10
        torch.cuda.synchronize()
    settle_s = time.perf_counter() - t_s
    warmup = 10 if args.warmup is None else args.warmup
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    graph = None
    if args.graph:
        # The timed steps as one HIP graph (captured on a side stream; the
        # step closures read `stream`, so they launch onto the capture
        # stream), replayed once: kernels back to back with no host launch
        # gaps, for workloads whose kernel is shorter than a host launch.
        launch_stream = stream
        cap = torch.cuda.Stream(dev)
        cap.wait_stream(launch_stream)
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.stream(cap):
            stream = cap
            with torch.cuda.graph(graph, stream=cap):
                for _ in range(args.steps):
                    step()
        stream = launch_stream
        graph.replay()  # one untimed replay
        torch.cuda.synchronize()
    # HIP events recorded on the stream the kernels are launched on.
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    if graph is not None:
        graph.replay()
    else:
        for _ in range(args.steps):
            step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps  # one call per step

    # Per-call distribution: one event pair around each call (at most 2000)
    # after the timed region, so the extra event records do not perturb it;
    # calls continue for at least DIST_S so that the graphics clock, sampled
    # every 10 ms, is read over a window of this kernel's sustained load.
    n_dist = min(2000, max(20, int(args.dist / max(ms * 1e-3, 1e-6))))
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
             for _ in range(n_dist)]
    t_d = time.perf_counter()
    for a, b in pairs:
        a.record(stream)
        step()
        b.record(stream)
    torch.cuda.synchronize()
    while time.perf_counter() - t_d < args.dist:
        for _ in range(10):
            step()
        torch.cuda.synchronize()
    t_d_end = time.perf_counter()
    clock.stop()
    per_launch = sorted(a.elapsed_time(b) for a, b in pairs)
    clk = sorted(clock.window(t_d, t_d_end))
    mhz = clk[len(clk) // 2] if len(clk) >= MIN_CLOCK_SAMPLES else None
    pw = sorted(clock.window(t_d, t_d_end, power=True))
    watts = pw[len(pw) // 2] if len(pw) >= MIN_CLOCK_SAMPLES else None

    if args.copy_calibration:
        src = torch.empty(COPY_BYTES // 4, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        for _ in range(COPY_REPS):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    comp = w.compulsory_bytes()
    gbps = comp / (ms * 1e-3) / 1e9
    # Stored counters describe the default schedule's kernel.
    traffic = measured_traffic(name, key) if args.persistent is None else None
    dist = [round(percentile(per_launch, f), 5) for f in (0.1, 0.5, 0.9)]
    props = torch.cuda.get_device_properties(dev)
    if cache:
        # Reading the cache from HBM bounds this path: GB/s against HBM peak.
        roofline = {
            "bound": "hbm",
            "achieved": round(gbps, 1),
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": round(gbps / HBM_PEAK_GBPS, 4),
            "traffic": traffic,
            "kernel_ms": round(ms, 5),
            "kernels_per_call": 1 if n_split == 1 else 2,
            "key_splits": n_split,
            "compulsory_bytes": comp,
            "tflops": round(tflops, 2),
            "launch_ms_p10_p50_p90": dist,
            "launches_sampled": len(per_launch),
        }
        if mhz:
            roofline["gfx_clock_mhz_median"] = round(mhz, 1)
            roofline["clock_samples"] = len(clk)
        result = {
            "metric": "attention decode against a K/V cache: GB/s of compulsory HBM bytes (1 GPU)",
            "value": round(gbps, 1),
            "unit": "GB/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": warmup,
            "ms_per_step": round(ms, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": w.dtype,
            "data": "synthetic",
            "config": {"workload": name, "B": w.B, "H": w.H, "Nq": w.Nq, "Nk": w.Nk, "d": w.d,
                       "causal": w.causal, "inputs": w.description},
            "roofline": roofline,
        }
    else:
        peak = MFMA_PEAK_TFLOPS[w.dtype]
        roofline = {
            "bound": "mfma",
            "achieved": round(tflops, 2),
            "peak": peak,
            "unit": "TFLOP/s",
            "frac": round(tflops / peak, 4),
            "traffic": traffic,
            "kernel_ms": round(ms, 5),
            "compulsory_bytes": comp,
            "compulsory_GBps": round(gbps, 1),
            "compulsory_frac_of_hbm_peak": round(gbps / HBM_PEAK_GBPS, 4),
            "launch_ms_p10_p50_p90": dist,
            "launches_sampled": len(per_launch),
        }
        if mhz:
            # The per-call median against the peak at the clock the card ran
            # during those same calls.  A fraction above 1 would mean the
            # clock reading does not describe the kernel's calls: then it is
            # left out.
            roofline["gfx_clock_mhz_median"] = round(mhz, 1)
            roofline["clock_samples"] = len(clk)
            if watts:
                roofline["socket_power_w_median"] = round(watts, 1)
            f = flops / (dist[1] * 1e-3) / 1e12 / (peak * mhz / PEAK_CLOCK_MHZ)
            if 0 < f <= 1:
                roofline["frac_at_measured_clock"] = round(f, 4)
        result = {
            "metric": ("attention fwd TFLOP/s and % of MFMA peak, e4m3 inputs (1 GPU)" if key == "fp8"
                       else "attention bwd TFLOP/s (2.5x the forward's FLOPs) and % of MFMA peak (1 GPU)"
                       if key == "bwd"
                       else "attention fwd TFLOP/s and % of MFMA peak, N=4096 d=128 fp16 (1 GPU)"),
            "value": round(tflops, 2),
            "unit": "TFLOP/s",
            "n_gpus": 1,
            "steps": args.steps,
            "warmup": warmup,
            "ms_per_step": round(ms, 5),
            "higher_is_better": True,
            "scaling": "weak",
            "vs_baseline": None,
            "dtype": w.dtype,
            "data": "synthetic",
            "config": {"workload": name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                       "causal": w.causal, "inputs": w.description},
            "roofline": roofline,
        }
        if args.persistent is not None:
            result["config"]["schedule"] = "persistent"
            result["config"]["num_workgroups"] = args.persistent
    result["device"] = {"name": props.name, "cus": props.multi_processor_count,
                        "arch": getattr(props, "gcnArchName", "")}
    result["timed_wall_s"] = round(wall, 4)
    result["launch"] = "hip_graph" if graph is not None else "stream"
    result["clock_settle"] = {"seconds": round(settle_s, 2), "calls": settle_calls,
                              "note": "untimed calls before the warm-up steps"}
    if args.cpu_budget > 0:
        if cache:
            result["cpu_baseline"] = cpu_baseline_cache(w, q, k, v, args.cpu_budget)
        elif key == "bwd":
            result["cpu_baseline"] = cpu_baseline_bwd(w, q, k, v, do, args.cpu_budget)
        elif key == "fp8":
            import oracle
            qx, kx, vx = (oracle.dequantize_fp8(x, s) for x, s in ((q, qs), (k, ks), (v, vs)))
            result["cpu_baseline"] = cpu_baseline(w, qx, kx, vx, args.cpu_budget)
        else:
            # The last timed call's outputs, compared with the oracle on the
            # rows the baseline computes.
            gpu_out = (o.float().cpu().numpy(), lse.cpu().numpy())
            result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_budget, gpu_out)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
