"""Throughput of one rank's share of Ring Attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]

One step = one fused launch of ra_rank_forward over the whole share (all c ring rounds,
causal skipping, GQA, lse) on seeded synthetic inputs already resident in HBM. The value
is unmasked TFLOP/s: 4*d FLOP per allowed score entry over the step time. Prints one
JSON line.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_F32_TFLOPS = 157.3       # MI355X dense fp32 matrix
METRIC = "attention TFLOP/s (unmasked) per rank share, 1 GPU; % of bf16 MFMA peak"
DEFAULT_WORKLOAD = "gqa64x8_d128_s128k_c16_zigzag_bf16"
ALSO_WORKLOADS = ["gqa32x8_d128_s32k_c8_zigzag_bf16"]
KERNEL_SOURCE = os.path.join(ROOT, "blockwise_ring_attention_amd", "csrc", "ra_fwd.hip")


def kernel_sha() -> str:
    return hashlib.sha256(open(KERNEL_SOURCE, "rb").read()).hexdigest()[:16]


def measured_traffic(workload: str, launch_ms: float):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were
    taken on the current kernel source; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    if rec.get("kernel_sha") != kernel_sha():
        return None
    return rec.get("hbm_bytes_per_launch")


def workload_numbers(w):
    from blockwise_ring_attention_amd import accounting as acc
    n = w.rows
    entries = acc.allowed_entries(w.c, w.rank, n, n, w.causal, w.zigzag)
    flop = acc.unmasked_flop(w.batch, w.hq, w.head_dim, entries)
    eb = 2 if w.dtype == "bf16" else 4
    nbytes = acc.algorithmic_bytes(w.batch, w.hq, w.hkv, n, n, w.head_dim, eb, w.c, w.rank, w.causal, w.zigzag,
                                   with_lse=w.with_lse)
    return flop, nbytes


def time_workload(w, steps: int, warmup: int, arrays=None):
    import torch
    import blockwise_ring_attention_amd as ra
    from blockwise_ring_attention_amd.inputs import make_inputs
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = arrays if arrays is not None else make_inputs(w)
    qd = torch.from_numpy(q).to("cuda", dt)
    kd = torch.from_numpy(k).to("cuda", dt)
    vd = torch.from_numpy(v).to("cuda", dt)
    del q, k, v
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda") if w.with_lse else None

    def step():
        ra.rank_forward(qd, kd, vd, w.c, w.rank, w.causal, w.zigzag, out=out, lse=lse, with_lse=w.with_lse)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    # Kernel time: HIP events on the stream the kernel is launched on (torch's current one).
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    del qd, kd, vd, out, lse
    torch.cuda.empty_cache()
    return wall / steps * 1e3, sum(launch_ms) / len(launch_ms), min(launch_ms)


def cpu_baseline(w, arrays, min_seconds: float = 10.0):
    """The oracle as it stands, timed on a bounded sample of the same workload: the first
    R query rows of batch 0 in head-major order, each as a full fp64 row against every
    key of the c blocks. R starts at 96 and doubles until one run of the oracle takes
    at least `min_seconds` (or covers the whole share); that run is reported."""
    import numpy as np
    import oracle
    q, k, v = arrays
    n = w.rows
    total_rows = w.hq * n
    count = 96
    while True:
        count = min(count, total_rows)
        idx = np.arange(count)
        rows = np.stack([np.zeros_like(idx), idx // n, idx % n], axis=1)
        t0 = time.perf_counter()
        oracle.rank_forward(q, k, v, w.c, w.rank, w.causal, w.zigzag, rows=rows)
        sec = time.perf_counter() - t0
        if sec >= min_seconds or count == total_rows:
            break
        count *= 2
    # unmasked work of the sampled rows: allowed keys per row
    ts = rows[:, 2]
    if w.causal:
        allowed = int((oracle.chunk_positions(w.rank, n, w.c, w.zigzag)[ts] + 1).sum())
    else:
        allowed = len(ts) * n * w.c
    flop = 4 * w.head_dim * allowed
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    try:
        from threadpoolctl import threadpool_info
        blas = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if blas:
            cores = max(blas)
    except Exception:
        pass
    return {
        "value": flop / sec / 1e12,
        "unit": "TFLOP/s",
        "cores": cores,
        "kind": "oracle",
        "sample": (f"first {count} query rows (head-major, batch 0) of {w.name}, each a full fp64 row "
                   f"against all {w.c * n} keys (masked entries computed and discarded); {sec:.1f} s wall; "
                   f"rate counts unmasked work only"),
        "seconds": sec,
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-also", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum length of the timed oracle run for cpu_baseline")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (to scale the "
                         "FETCH_SIZE/WRITE_SIZE counters against a kernel of known traffic)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one rank's share on one GPU; --gpus {args.gpus} is not supported "
              "(this build has no multi-GPU path)", file=sys.stderr)
        sys.exit(2)

    import torch
    if args.calibrate_copy:
        n = args.calibrate_copy * (1 << 20) // 4
        src = torch.ones(n, dtype=torch.float32, device="cuda")
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"calibrate_copy_bytes": n * 4, "copies": 3}), flush=True)
        return
    from blockwise_ring_attention_amd import _binding
    from blockwise_ring_attention_amd.inputs import WORKLOADS
    if not os.path.exists(_binding.LIB_PATH):
        from blockwise_ring_attention_amd.csrc import build
        build.build()
    from blockwise_ring_attention_amd.inputs import make_inputs
    w = WORKLOADS[args.workload]
    flop, nbytes = workload_numbers(w)
    arrays = make_inputs(w)
    ms_step, ms_launch, ms_min = time_workload(w, args.steps, args.warmup, arrays)
    value = flop / (ms_step * 1e-3) / 1e12
    peak = PEAK_BF16_TFLOPS if w.dtype == "bf16" else PEAK_F32_TFLOPS
    achieved = flop / (ms_launch * 1e-3) / 1e12
    traffic = measured_traffic(w.name, ms_launch)
    line = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded Gaussian Q/K/V, inputs resident in HBM)",
        "config": {"workload": w.name, "batch": w.batch, "hq": w.hq, "hkv": w.hkv, "head_dim": w.head_dim,
                   "seq": w.seq, "c": w.c, "rank": w.rank, "causal": w.causal, "zigzag": w.zigzag,
                   "query_rows": w.rows, "lse": w.with_lse, "parallelism": "one rank's share, 1 GPU"},
        "pct_of_peak": round(100 * value / peak, 2),
        "unmasked_flop": flop,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic,
                     "algorithmic_bytes": nbytes, "kernel_ms_avg": round(ms_launch, 4),
                     "kernel_ms_min": round(ms_min, 4)},
    }
    if not args.no_also:
        also = []
        for name in ALSO_WORKLOADS:
            wa = WORKLOADS[name]
            fa, _ = workload_numbers(wa)
            ms_a, ml_a, _ = time_workload(wa, args.steps, args.warmup)
            also.append({"workload": name, "value": round(fa / (ms_a * 1e-3) / 1e12, 2), "ms_per_step": round(ms_a, 4),
                         "pct_of_peak": round(100 * fa / (ms_a * 1e-3) / 1e12 / PEAK_BF16_TFLOPS, 2)})
        line["also"] = also
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, arrays, args.cpu_seconds)
    torch.cuda.synchronize()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
