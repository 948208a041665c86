"""Benchmark of the gfx950 FlashAttention forward pass on one GPU.

One step = one forward pass (scores, online softmax, P V, O and LSE written)
over the whole workload, inputs already resident in HBM.  Prints one JSON
line: throughput in TFLOP/s (4*B*H*N^2*d matrix FLOPs per step, halved under
the causal mask), the roofline of the kernel against the MI355X dense MFMA
peak, and the fp64 CPU oracle timed on a bounded sample of the same workload.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# MI355X published dense peaks (TFLOP/s) and HBM bandwidth (GB/s).
MFMA_PEAK_TFLOPS = {"f16": 2516.6, "bf16": 2516.6, "f32": 157.3}
HBM_PEAK_GBPS = 8000.0
KERNEL_SOURCE = os.path.join(ROOT, "io_aware_tiled_08_amd", "csrc", "fa_fwd_f16.hip")
PROFILES = os.path.join(ROOT, "profiles")


def kernel_source_digest() -> str:
    with open(KERNEL_SOURCE, "rb") as f:
        return hashlib.sha256(f.read()).hexdigest()


def measured_traffic(workload: str):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when there is none or the kernel source changed since it was taken."""
    path = os.path.join(PROFILES, f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("kernel_source_sha256") != kernel_source_digest():
        return None
    return t.get("hbm_bytes_per_launch")


def cpu_baseline(w, q, k, v, budget_s: float):
    """Times the fp64 oracle on whole heads of the workload until the budget
    is spent (at least one head)."""
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()
                       if p.get("user_api") == "blas"] or [1])
    except Exception:  # threadpoolctl missing: numpy's BLAS default
        threads = len(os.sched_getaffinity(0))
    heads = [(b, h) for b in range(w.B) for h in range(w.H)]
    done = 0
    t0 = time.perf_counter()
    for b, h in heads:
        sl = (slice(b, b + 1), slice(h, h + 1))
        oracle.attention_forward(q[sl], k[sl], v[sl], w.scale, w.causal)
        done += 1
        if time.perf_counter() - t0 >= budget_s:
            break
    el = time.perf_counter() - t0
    from io_aware_tiled_08_amd.workloads import metric_flops
    flops = metric_flops(1, 1, w.N, w.d, w.causal) * done
    return {
        "value": flops / el / 1e12,
        "unit": "TFLOP/s",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{done} of {len(heads)} (b,h) heads of {w.name}, all {w.N} query rows "
                  f"each, fp64 numpy, {el:.1f} s",
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default=None)
    ap.add_argument("--cpu-budget", type=float, default=12.0,
                    help="seconds of oracle time for cpu_baseline (0 = skip)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (got --gpus {args.gpus}): the forward pass "
              "shards by (batch, head) with no communication, and this build measures "
              "one GPU's share.", file=sys.stderr)
        sys.exit(2)

    import torch

    from io_aware_tiled_08_amd import binding, flash_attn_fwd
    from io_aware_tiled_08_amd import workloads as W
    if not os.path.exists(binding.library_path()):
        from io_aware_tiled_08_amd.build import build_library
        build_library()

    name = args.workload or W.HEADLINE
    w = W.WORKLOADS[name]
    q, k, v = W.workload_inputs(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (x.to(dev) for x in (q, k, v))
    o = torch.empty_like(qd)
    lse = torch.empty((w.B, w.H, w.N), dtype=torch.float32, device=dev)
    stream = torch.cuda.current_stream(dev)

    def step():
        flash_attn_fwd(qd, kd, vd, o, lse, scale=w.scale, causal=w.causal, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    start.record(stream)
    for _ in range(args.steps):
        step()
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms = start.elapsed_time(end) / args.steps

    flops = w.flops()
    tflops = flops / (ms * 1e-3) / 1e12
    peak = MFMA_PEAK_TFLOPS[w.dtype]
    traffic = measured_traffic(name)
    roofline = {
        "bound": "mfma",
        "achieved": round(tflops, 2),
        "peak": peak,
        "unit": "TFLOP/s",
        "frac": round(tflops / peak, 4),
        "traffic": traffic,
        "compulsory_bytes": w.compulsory_bytes(),
        "compulsory_GBps": round(w.compulsory_bytes() / (ms * 1e-3) / 1e9, 1),
    }
    props = torch.cuda.get_device_properties(dev)
    result = {
        "metric": "attention fwd TFLOP/s and % of MFMA peak, N=4096 d=128 fp16 (1 GPU)",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic",
        "config": {"workload": name, "B": w.B, "H": w.H, "N": w.N, "d": w.d,
                   "causal": w.causal, "inputs": w.description},
        "roofline": roofline,
        "device": {"name": props.name, "cus": props.multi_processor_count,
                   "arch": getattr(props, "gcnArchName", "")},
        "timed_wall_s": round(wall, 4),
    }
    if args.cpu_budget > 0:
        result["cpu_baseline"] = cpu_baseline(w, q, k, v, args.cpu_budget)
    else:
        result["cpu_baseline"] = None
    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
