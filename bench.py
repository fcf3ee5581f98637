"""Throughput of one rank's share of Ring Attention on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--no-cpu-baseline]
                    [--no-also] [--no-per-round] [--balance]

One step = one fused launch of ra_rank_forward over the whole share (all c ring rounds,
causal skipping, GQA, lse) on seeded synthetic inputs already resident in HBM. The value
is unmasked TFLOP/s: 4*d FLOP per allowed score entry over the step time. Prints one
JSON line; it also carries the streamed form of the same share ("per_round": one launch
per ring round, folded into the running result by the kernel's own epilogue with the
running out in fp32 or in bf16, and plain launches with a separate ra_merge per round).
``--balance`` instead times every rank of the workload with contiguous and with zigzag
chunks and prints that sweep.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6     # MI355X dense bf16 MFMA: 256 CU x 4096 FLOP/clk x 2.4 GHz
PEAK_F32_TFLOPS = 157.3       # MI355X dense fp32 matrix
METRIC = "attention TFLOP/s (unmasked) per rank share, 1 GPU; % of bf16 MFMA peak"
DEFAULT_WORKLOAD = "gqa64x8_d128_s128k_c16_zigzag_bf16"
ALSO_WORKLOADS = ["gqa32x8_d128_s32k_c8_zigzag_bf16", "mha16_b2_d128_s64k_c8_noncausal_outliers_bf16",
                  "mha_d64_s4k_c4_zigzag_fp32", "gqa32x8_d128_s32k_c8_zigzag_fp32"]
MIN_TIMED_MS = 200.0   # short workloads get more steps so the timed region spans this much
WARMUP_MS = 1000.0     # warmup runs at least this long: the chip's clock ramps up under load
KERNEL_SOURCES = [os.path.join(ROOT, "blockwise_ring_attention_amd", "csrc", f)
                  for f in ("ra_fwd.hip", "ra_internal.h")]


XGMI_LINK_GBPS = 153.0         # one MI355X xGMI link, one direction (spec figure)
PAGES_H100_TFLOPS = 989.0     # the pages' break-even arithmetic: H100 dense bf16 ...
PAGES_NVLINK_GBPS = 450.0     # ... over NVLink


class ClockSampler:
    """Polls the GPU's graphics clock (and socket power) through amdsmi's gpu_metrics
    while the timed launches run, from a daemon thread every `period_s`. The device is
    matched to torch's by PCI address. Any failure leaves the result with an "error"
    entry instead of figures: the clock is reported, never required."""

    def __init__(self, device_index: int = 0, period_s: float = 0.02):
        self.device_index = device_index
        self.period_s = period_s
        self.samples, self.xcd, self.power = [], [], []
        self.error = None
        self._handle = None
        self._stop = None
        self._thread = None

    def _open(self):
        import amdsmi
        import torch
        amdsmi.amdsmi_init()
        props = torch.cuda.get_device_properties(self.device_index)
        want = (int(props.pci_domain_id), int(props.pci_bus_id), int(props.pci_device_id))
        handles = amdsmi.amdsmi_get_processor_handles()
        for h in handles:
            bdf = amdsmi.amdsmi_get_gpu_device_bdf(h)          # "DDDD:BB:DD.F"
            dom, bus, rest = bdf.split(":")
            if (int(dom, 16), int(bus, 16), int(rest.split(".")[0], 16)) == want:
                return h
        if len(handles) == 1:
            return handles[0]
        raise RuntimeError(f"no amdsmi device at PCI {want} among {len(handles)}")

    def _read(self):
        import amdsmi
        m = amdsmi.amdsmi_get_gpu_metrics_info(self._handle)
        clks = m.get("current_gfxclks")
        xcd = [int(x) for x in clks if isinstance(x, (int, float)) and 0 < x < 10000] if isinstance(clks, list) else []
        one = m.get("current_gfxclk")
        if not isinstance(one, (int, float)) or not 0 < one < 10000:
            one = sum(xcd) / len(xcd) if xcd else None
        pw = m.get("current_socket_power")
        if not isinstance(pw, (int, float)) or not 0 < pw < 100000:
            pw = m.get("average_socket_power")
        return one, xcd, pw if isinstance(pw, (int, float)) and 0 < pw < 100000 else None

    def __enter__(self):
        import threading
        try:
            self._handle = self._open()
            self._read()
        except Exception as e:   # noqa: BLE001 - report, never fail the bench
            self.error = f"{type(e).__name__}: {e}"
            return self
        self._stop = threading.Event()

        def loop():
            while not self._stop.is_set():
                try:
                    one, xcd, pw = self._read()
                    if one is not None:
                        self.samples.append(one)
                    if xcd:
                        self.xcd.append(xcd)
                    if pw is not None:
                        self.power.append(pw)
                except Exception as e:   # noqa: BLE001
                    self.error = f"{type(e).__name__}: {e}"
                    return
                self._stop.wait(self.period_s)

        self._thread = threading.Thread(target=loop, daemon=True)
        self._thread.start()
        return self

    def __exit__(self, *exc):
        if self._thread is not None:
            self._stop.set()
            self._thread.join()
        return False

    def result(self):
        if not self.samples:
            return {"error": self.error or "no samples"}
        r = {"gfx_mhz_median": float(np.median(self.samples)), "gfx_mhz_mean": round(float(np.mean(self.samples)), 1),
             "gfx_mhz_min": float(np.min(self.samples)), "gfx_mhz_max": float(np.max(self.samples)),
             "samples": len(self.samples),
             "source": f"amdsmi gpu_metrics current_gfxclk, polled every {self.period_s * 1e3:.0f} ms "
                       "during the timed launches"}
        if self.xcd:
            width = min(len(x) for x in self.xcd)
            r["per_xcd_mhz_median"] = [float(np.median([x[i] for x in self.xcd])) for i in range(width)]
        if self.power:
            r["socket_power_w_mean"] = round(float(np.mean(self.power)), 1)
        if self.error:
            r["error"] = self.error
        return r


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.lower().startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    import platform
    return platform.processor() or "unknown"


def kernel_sha() -> str:
    """sha256[:16] over the forward kernel's sources (the kernel file, then its header)."""
    h = hashlib.sha256()
    for f in KERNEL_SOURCES:
        h.update(open(f, "rb").read())
    return h.hexdigest()[:16]


def library_sha() -> str:
    """sha256[:16] of the built library the bench loads (the compiled kernels themselves:
    a source edit that leaves the shipped build unchanged, such as a diagnostic-only
    switch, leaves it unchanged too)."""
    from blockwise_ring_attention_amd import _binding
    h = hashlib.sha256()
    with open(_binding.LIB_PATH, "rb") as f:
        h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload: str, launch_ms: float):
    """HBM bytes per launch from the committed rocprofv3 counter runs, if they were
    taken on the library the bench loads; else None."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path))
    try:
        if rec.get("library_sha") != library_sha():
            return None
    except OSError:
        return None
    return rec.get("hbm_bytes_per_launch")


def workload_numbers(w):
    from blockwise_ring_attention_amd import accounting as acc
    from blockwise_ring_attention_amd.inputs import make_doc_start
    n = w.rows
    eb = 2 if w.dtype == "bf16" else 4
    ds = make_doc_start(w)
    if ds is not None:
        entries = acc.doc_allowed_entries(w.c, w.rank, n, w.zigzag, ds)
        kv_rows = acc.doc_needed_kv_rows(w.c, w.rank, n, w.zigzag, ds)
        io = 2 * w.batch * w.hq * n * w.head_dim * eb + (4 * w.batch * w.hq * n if w.with_lse else 0)
        nbytes = io + 2 * w.batch * w.hkv * kv_rows * w.head_dim * eb
    else:
        entries = acc.allowed_entries(w.c, w.rank, n, n, w.causal, w.zigzag)
        nbytes = acc.algorithmic_bytes(w.batch, w.hq, w.hkv, n, n, w.head_dim, eb, w.c, w.rank, w.causal, w.zigzag,
                                       with_lse=w.with_lse)
    flop = acc.unmasked_flop(w.batch, w.hq, w.head_dim, entries)
    return flop, nbytes


def time_workload(w, steps: int, warmup: int, arrays=None, clock=None, warmup_ms: float = WARMUP_MS):
    """Time `steps` launches after at least `warmup` untimed ones, and after as many more
    as it takes for the warmup to last `warmup_ms` (the graphics clock settles under load
    over tens of launches). Returns (ms per step by wall clock, mean / min / median kernel
    ms by HIP events, warmup steps run)."""
    import torch
    import blockwise_ring_attention_amd as ra
    qd, kd, vd = _device_inputs(w, arrays)
    fwd = _forward_fn(w)
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda") if w.with_lse else None

    def step():
        fwd(qd, kd, vd, out=out, lse=lse, with_lse=w.with_lse)

    # the first launch also loads the library's code objects: it does not count as warmup time
    step()
    torch.cuda.synchronize()
    done = 1
    t_w = time.perf_counter()
    while done < warmup or (time.perf_counter() - t_w) * 1e3 < warmup_ms:
        step()
        done += 1
        if done >= warmup:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    # Kernel time: HIP events on the stream the kernel is launched on (torch's current one).
    stream = torch.cuda.current_stream()
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    if clock is not None:
        clock.__enter__()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record(stream)
        step()
        e1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    if clock is not None:
        clock.__exit__(None, None, None)
    launch_ms = [e0.elapsed_time(e1) for e0, e1 in ev]
    del qd, kd, vd, out, lse
    torch.cuda.empty_cache()
    return (wall / steps * 1e3, sum(launch_ms) / len(launch_ms), min(launch_ms), float(np.median(launch_ms)),
            done)


def time_workload_min(w, steps: int, warmup: int, arrays=None, min_ms: float = MIN_TIMED_MS, clock=None,
                      warmup_ms: float = WARMUP_MS):
    """time_workload, run again with more steps when `steps` launches last less than
    `min_ms`. Returns its four timing figures, the step count of the run reported and its
    warmup steps."""
    r = time_workload(w, steps, warmup, arrays, warmup_ms=warmup_ms)
    if steps * r[0] < min_ms or clock is not None:
        steps = max(steps, int(np.ceil(min_ms / r[0])))
        r = time_workload(w, steps, warmup, arrays, clock=clock, warmup_ms=warmup_ms)
    return (*r[:4], steps, r[4])


def _device_inputs(w, arrays):
    import torch
    from blockwise_ring_attention_amd.inputs import make_inputs
    dt = torch.bfloat16 if w.dtype == "bf16" else torch.float32
    q, k, v = arrays if arrays is not None else make_inputs(w)
    return (torch.from_numpy(q).to("cuda", dt), torch.from_numpy(k).to("cuda", dt),
            torch.from_numpy(v).to("cuda", dt))


def _forward_fn(w):
    """ra.rank_forward for the workload, or ra.rank_forward_doc with its document layout
    (uploaded once) when it has one; same call signature either way."""
    import torch
    import blockwise_ring_attention_amd as ra
    from blockwise_ring_attention_amd.inputs import make_doc_start
    ds = make_doc_start(w)
    if ds is None:
        return lambda q, k, v, t0=0, t1=None, **kw: ra.rank_forward(q, k, v, w.c, w.rank, w.causal, w.zigzag,
                                                                    t0, t1, **kw)
    dd = torch.from_numpy(ds).to("cuda")
    return lambda q, k, v, t0=0, t1=None, **kw: ra.rank_forward_doc(q, k, v, dd, w.c, w.rank, w.zigzag, t0, t1, **kw)


def _accumulate_fn(w):
    """ra.rank_forward_accumulate for the workload (with its document layout if any)."""
    import torch
    import blockwise_ring_attention_amd as ra
    from blockwise_ring_attention_amd.inputs import make_doc_start
    ds = make_doc_start(w)
    dd = torch.from_numpy(ds).to("cuda") if ds is not None else None
    return lambda q, k, v, out, lse, t0, t1: ra.rank_forward_accumulate(q, k, v, out, lse, w.c, w.rank, w.causal,
                                                                        w.zigzag, t0, t1, doc_start=dd)


def time_per_round(w, steps: int, warmup: int, arrays=None, mode: str = "accumulate"):
    """The streamed form of the same share, as a live ring rank runs it: one launch per
    ring round (rounds [t, t+1)), in ring order, the running (out, lse) kept in HBM.
    Modes: "accumulate" folds every round into an fp32 running out inside the kernel's
    epilogue (ra_rank_forward_accumulate, starting from lse = -inf) and rounds it to the
    input dtype once at the end; "accumulate_bf16" keeps the running out in bf16 (round 0
    a plain launch); "merge" runs plain launches and merges each later round's partial in
    place with ra_merge; "accumulate_graph" is "accumulate" captured once in a HIP graph
    and replayed, as a rank that issues the same c launches every step would run it.
    One step = all c rounds (with the fill and the final rounding). Returns step ms,
    per-round kernel ms, per-merge ms (from one event-instrumented step; none for the
    graph) and the max abs difference of the streamed result from the fused launch."""
    import torch
    import blockwise_ring_attention_amd as ra
    graph_mode = mode == "accumulate_graph"
    if graph_mode:
        mode = "accumulate"
    qd, kd, vd = _device_inputs(w, arrays)
    fwd = _forward_fn(w)
    accf = _accumulate_fn(w)
    acc = torch.empty_like(qd)
    acc32 = torch.empty(qd.shape, dtype=torch.float32, device="cuda") if mode == "accumulate" else None
    acc_lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    part = torch.empty_like(qd) if mode == "merge" else None
    part_lse = torch.empty_like(acc_lse) if mode == "merge" else None
    c = w.c

    def launch(t):
        if mode == "accumulate":
            accf(qd, kd, vd, acc32, acc_lse, t, t + 1)
        elif t == 0:
            fwd(qd, kd, vd, 0, 1, out=acc, lse=acc_lse)
        elif mode == "merge":
            fwd(qd, kd, vd, t, t + 1, out=part, lse=part_lse)
        else:
            accf(qd, kd, vd, acc, acc_lse, t, t + 1)

    def merge():
        ra.merge(acc, acc_lse, part, part_lse, out=acc, lse=acc_lse)

    has_merge = mode == "merge"

    def step():
        if mode == "accumulate":
            acc_lse.fill_(float("-inf"))
        for t in range(c):
            launch(t)
            if t > 0 and has_merge:
                merge()
        if mode == "accumulate":
            acc.copy_(acc32)

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    run = step
    if graph_mode:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            step()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            step()
        run = graph.replay
        run()
        torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(steps):
        run()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / steps
    if graph_mode:
        round_ms, merge_ms = [], []
        return _streamed_result(fwd, qd, kd, vd, acc, acc_lse, ms_step, round_ms, merge_ms)
    # one instrumented step: an event pair around every launch and every merge
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(c)]
    if mode == "accumulate":
        acc_lse.fill_(float("-inf"))
    for t in range(c):
        ev[t][0].record(stream)
        launch(t)
        ev[t][1].record(stream)
        if t > 0 and has_merge:
            ev[t][2].record(stream)
            merge()
            ev[t][3].record(stream)
    if mode == "accumulate":
        acc.copy_(acc32)
    torch.cuda.synchronize()
    round_ms = [ev[t][0].elapsed_time(ev[t][1]) for t in range(c)]
    merge_ms = [ev[t][2].elapsed_time(ev[t][3]) for t in range(1, c)] if has_merge else []
    return _streamed_result(fwd, qd, kd, vd, acc, acc_lse, ms_step, round_ms, merge_ms)


def _streamed_result(fwd, qd, kd, vd, acc, acc_lse, ms_step, round_ms, merge_ms):
    """The streamed result against one fused launch: max abs differences of out and lse."""
    import torch
    fused, fused_lse = fwd(qd, kd, vd, with_lse=True)
    torch.cuda.synchronize()
    diff = (acc.float() - fused.float()).abs().max().item()
    fin = torch.isfinite(fused_lse)
    lse_diff = (acc_lse[fin] - fused_lse[fin]).abs().max().item() if bool(fin.any()) else 0.0
    del fused, fused_lse
    torch.cuda.empty_cache()
    return ms_step, round_ms, merge_ms, diff, lse_diff


def balance_sweep(w, steps: int, warmup: int, warmup_ms: float = WARMUP_MS):
    """Every rank r = 0..c-1 of the workload, once with contiguous chunks and once with
    the zigzag pairing (causal), each a fused launch: ms per rank and the spread. Q is the
    same array for every rank (its values do not change the work). Each rank is timed
    over at least MIN_TIMED_MS of launches."""
    import dataclasses
    import torch
    from blockwise_ring_attention_amd import accounting as acc
    from blockwise_ring_attention_amd.inputs import make_doc_start, make_inputs
    arrays = make_inputs(w)
    ds = make_doc_start(w)
    res = {}
    for zig in (False, True):
        ranks = []
        for r in range(w.c):
            wr = dataclasses.replace(w, rank=r, zigzag=zig)
            ms, ml, mn, _, steps_r, _ = time_workload_min(wr, steps, warmup, arrays, warmup_ms=warmup_ms)
            if ds is None:
                e = acc.allowed_entries(w.c, r, w.rows, w.rows, True, zig)
            else:
                e = acc.doc_allowed_entries(w.c, r, w.rows, zig, ds)
            flop = acc.unmasked_flop(w.batch, w.hq, w.head_dim, e)
            rec = {"rank": r, "kernel_ms": round(ml, 4), "tflops": round(flop / (ml * 1e-3) / 1e12, 1),
                   "allowed_entries_per_head": e, "steps": steps_r}
            if ds is None:
                rec["kv_blocks_with_work"] = sum(
                    1 for j in range(w.c) if acc.block_allowed(w.c, r, j, w.rows, w.rows, True, zig) > 0)
            ranks.append(rec)
        times = [x["kernel_ms"] for x in ranks]
        res["zigzag" if zig else "contiguous"] = {
            "ranks": ranks, "max_ms": max(times), "min_ms": min(times),
            "max_over_min": round(max(times) / min(times), 3),
            "ring_round_ms_bound": round(max(times), 4)}
        torch.cuda.empty_cache()
    return res


def break_even_context(w, kernel_ms: float, tflops: float):
    """The pages' compute/transfer break-even, quoted as hardware arithmetic (not a
    measured result or a target), beside the same arithmetic for this workload at the
    measured rate ("What do you do about long sequences and sparse models?", section
    "When is the ring actually free?": a block of c tokens costs 4 d c^2 FLOP against
    4 c d bytes to send, so the send hides when c >= F / B)."""
    eb = 2 if w.dtype == "bf16" else 4
    block_bytes = 2 * w.batch * w.hkv * w.rows * w.head_dim * eb        # one K and V block
    round_ms = kernel_ms / w.c                                          # mean ring round of the fused launch
    ctx = {
        "pages_break_even_tokens": round(PAGES_H100_TFLOPS * 1e12 / (PAGES_NVLINK_GBPS * 1e9), 1),
        "pages_arithmetic": f"{PAGES_H100_TFLOPS:.0f} TFLOP/s (H100) / {PAGES_NVLINK_GBPS:.0f} GB/s (NVLink) "
                            "= tokens per block at which a block's compute hides its transfer (single head)",
        "same_arithmetic_mi355x_peak_one_xgmi_link_tokens": round(PEAK_BF16_TFLOPS * 1e12 / (XGMI_LINK_GBPS * 1e9), 1),
        "same_arithmetic_measured_rate_one_xgmi_link_tokens": round(tflops * 1e12 / (XGMI_LINK_GBPS * 1e9), 1),
        "mean_round_ms": round(round_ms, 4),
        "kv_block_bytes": block_bytes,
        "link_gbps_needed_to_hide_a_round": round(block_bytes / (round_ms * 1e-3) / 1e9, 1),
        "xgmi_link_gbps": XGMI_LINK_GBPS,
    }
    if w.causal and w.zigzag and w.c > 1:
        # a non-local zigzag round holds 2 m^2 of the share's (2c-1) m^2 + m(m+1) entries
        m = w.rows // 2
        frac = 2 * m * m / ((2 * w.c - 1) * m * m + m * (m + 1))
        ctx["nonlocal_round_ms_at_measured_rate"] = round(kernel_ms * frac, 4)
        ctx["link_gbps_needed_nonlocal_round"] = round(block_bytes / (kernel_ms * frac * 1e-3) / 1e9, 1)
        # m >= F Hkv / (B Hq): the zigzag GQA form of the same inequality
        ctx["min_chunk_tokens_to_hide_on_one_link"] = round(
            tflops * 1e12 * w.hkv / (XGMI_LINK_GBPS * 1e9 * w.hq), 1)
    return ctx


def sustain_run(w, seconds: float, flop: float, buckets: int = 12):
    """Launch the workload back to back for `seconds`, starting from an idle GPU, timing
    every launch with HIP events and sampling the clock and power every 20 ms: the
    throughput of each consecutive slice of the run, and the samples of that slice."""
    import torch
    qd, kd, vd = _device_inputs(w, None)
    fwd = _forward_fn(w)
    out = torch.empty_like(qd)
    lse = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    fwd(qd, kd, vd, out=out, lse=lse)
    torch.cuda.synchronize()
    t_one = time.perf_counter()
    fwd(qd, kd, vd, out=out, lse=lse)
    torch.cuda.synchronize()
    n = max(buckets, int(seconds / max(1e-4, time.perf_counter() - t_one)))
    time.sleep(2.0)   # idle first
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(n)]
    clock = ClockSampler(period_s=0.02)
    stamps = []
    clock.__enter__()
    t0 = time.perf_counter()
    for e0, e1 in ev:
        e0.record()
        fwd(qd, kd, vd, out=out, lse=lse)
        e1.record()
    torch.cuda.synchronize()
    clock.__exit__(None, None, None)
    ms = np.array([a.elapsed_time(b) for a, b in ev])
    per = n // buckets
    rows = []
    t = 0.0
    for i in range(buckets):
        seg = ms[i * per:(i + 1) * per]
        rows.append({"launches": [i * per, (i + 1) * per - 1], "start_s": round(t / 1e3, 3),
                     "kernel_ms": round(float(seg.mean()), 4), "tflops": round(flop / (seg.mean() * 1e-3) / 1e12, 1)})
        t += float(seg.sum())
    res = {"launches": n, "seconds": round(time.perf_counter() - t0, 2), "slices": rows,
           "clock": clock.result(), "clock_samples": [round(x) for x in clock.samples],
           "power_samples": [round(x) for x in clock.power]}
    del qd, kd, vd, out, lse
    torch.cuda.empty_cache()
    return res


def summarize_timeline(rec, kernel_ms: float):
    """One recorded launch of the timeline build: rec is [workgroups, 8] int64 (entry,
    after the first stage's barrier, end of the stage loop, end: ticks of the constant
    100 MHz clock; HW_ID; XCC_ID; stages of the loop; tile)."""
    n = int(np.count_nonzero(rec[:, 0]))
    rec = rec[:n]
    t = (rec[:, :4] - rec[:, 0].min()).astype(np.float64) / 100.0   # microseconds
    folded = rec[:, 1] != 0   # tiles that folded a stage
    hw = rec[:, 4]
    xcc = rec[:, 5] & 0xF
    cu = xcc * 4096 + (hw >> 8 & 0xFF)   # XCC, SE, SH and CU fields of HW_ID
    stages = rec[:, 6].astype(np.float64)
    prologue = (t[:, 1] - t[:, 0])[folded]
    tail = (t[:, 3] - t[:, 2])[folded]
    gaps, cu_end = [], {}
    for c in np.unique(cu):
        idx = np.where(cu == c)[0]
        idx = idx[np.argsort(t[idx, 0])]
        gaps.extend(t[idx[1:], 0] - t[idx[:-1], 3])
        cu_end[int(c)] = t[idx, 3].max()
    gaps = np.array(gaps) if gaps else np.zeros(1)
    xcds = []
    for x in range(8):
        m = xcc == x
        ends = [e for c, e in cu_end.items() if c // 4096 == x]
        long_ = m & folded & (stages >= 8)
        xcds.append({"xcd": x, "workgroups": int(m.sum()), "cus": len(ends),
                     "end_us": round(float(max(ends)), 1) if ends else None,
                     "cu_end_spread_us": round(float(max(ends) - min(ends)), 1) if ends else None,
                     "us_per_stage": round(float((t[long_, 2] - t[long_, 1]).sum() / stages[long_].sum()), 4)
                     if long_.any() else None})
    ends = np.array([x["end_us"] for x in xcds if x["end_us"] is not None])
    span = float(t[:, 3].max())
    return {"kernel_ms": round(kernel_ms, 4), "span_us": round(span, 1), "workgroups": n,
            "cus": len(cu_end),
            # workgroup i ran on XCD (i + o) mod 8 for one o (the round-robin's starting
            # XCD, where the previous dispatch left off), else None
            "xcd_offset": int(xcc[0]) if np.array_equal(xcc, (np.arange(n) + xcc[0]) % 8) else None,
            "xcd": xcds,
            "xcd_end_mean_us": round(float(ends.mean()), 1),
            "slowest_xcd_over_mean": round(float(ends.max() / ends.mean() - 1), 4),
            "slowest_xcd_over_fastest": round(float(ends.max() / ends.min() - 1), 4),
            "prologue_us_median": round(float(np.median(prologue)), 2),
            "tail_us_median": round(float(np.median(tail)), 2),
            "relaunch_gap_us_median": round(float(np.median(gaps)), 2),
            "relaunch_gap_us_p90": round(float(np.percentile(gaps, 90)), 2),
            "tiles_per_cu": round(n / max(1, len(cu_end)), 2)}


def timeline_run(w, launches: int, warmup_ms: float = WARMUP_MS):
    """The workload through the diagnostic build that records, per workgroup of the bf16
    kernel, the constant 100 MHz clock at entry, after the first stage's barrier, at the
    end of the stage loop and after the epilogue's stores, with HW_ID and XCC_ID. Warm
    launches come first (nothing recorded), then `launches` bursts of back-to-back
    launches, each at least 200 ms long, into the recording buffer: every launch of a
    burst overwrites it, so it holds the burst's last launch, taken under steady load (a
    launch that follows an idle gap runs while the clock is still settling). The output
    must equal the shipped library's bit for bit."""
    import ctypes
    import torch
    from blockwise_ring_attention_amd import _binding
    from blockwise_ring_attention_amd.csrc import build
    if w.dtype != "bf16":
        raise SystemExit("--timeline records the bf16 kernel")
    qd, kd, vd = _device_inputs(w, None)
    fwd = _forward_fn(w)
    out_ref = torch.empty_like(qd)
    lse_ref = torch.empty(qd.shape[:3], dtype=torch.float32, device="cuda")
    fwd(qd, kd, vd, out=out_ref, lse=lse_ref)   # the shipped library
    torch.cuda.synchronize()
    path = build.ablation_path("timeline")
    lib = _binding.use_library(path)
    lib.ra_diag_timeline.argtypes = [ctypes.c_void_p, ctypes.c_int]
    lib.ra_diag_timeline.restype = ctypes.c_int
    out = torch.empty_like(qd)
    lse = torch.empty_like(lse_ref)
    t_w = time.perf_counter()
    warm = 0
    while warm < 3 or (time.perf_counter() - t_w) * 1e3 < warmup_ms:
        fwd(qd, kd, vd, out=out, lse=lse)
        warm += 1
        torch.cuda.synchronize()
    per_launch_ms = (time.perf_counter() - t_w) * 1e3 / warm
    burst = max(2, int(np.ceil(200.0 / max(per_launch_ms, 1e-3))))
    cap = 1 << 16
    buf = torch.zeros((cap, 8), dtype=torch.int64, device="cuda")
    rows = []
    for _ in range(launches):
        buf.zero_()
        torch.cuda.synchronize()
        assert lib.ra_diag_timeline(ctypes.c_void_p(buf.data_ptr()), cap) == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        for i in range(burst):
            if i == burst - 1:
                e0.record()
            fwd(qd, kd, vd, out=out, lse=lse)
        e1.record()
        torch.cuda.synchronize()
        assert lib.ra_diag_timeline(None, 0) == 0
        rows.append({"burst": burst, **summarize_timeline(buf.cpu().numpy(), e0.elapsed_time(e1))})
    identical = bool(torch.equal(out, out_ref) and torch.equal(lse, lse_ref))
    del qd, kd, vd, out, lse, out_ref, lse_ref, buf
    torch.cuda.empty_cache()
    return {"library": os.path.relpath(path, ROOT), "warm_launches": warm, "identical_to_shipped": identical,
            "launches": rows}


def cpu_sample(w, count: int):
    """`count` query rows of batch 0 spread evenly over the share (head-major order), so
    light and heavy rows of a causal share enter in proportion, and the unmasked FLOP of
    those rows (4 d per allowed key)."""
    import numpy as np
    import oracle
    from blockwise_ring_attention_amd.inputs import make_doc_start
    n = w.rows
    total_rows = w.hq * n
    count = min(count, total_rows)
    idx = (np.arange(count, dtype=np.int64) * total_rows) // count
    rows = np.stack([np.zeros_like(idx), idx // n, idx % n], axis=1)
    ts = rows[:, 2]
    ds = make_doc_start(w)
    if ds is not None:
        p = oracle.chunk_positions(w.rank, n, w.c, w.zigzag)[ts]
        allowed = int(np.clip(p - np.maximum(ds[p], 0) + 1, 0, None).sum())
    elif w.causal:
        allowed = int((oracle.chunk_positions(w.rank, n, w.c, w.zigzag)[ts] + 1).sum())
    else:
        allowed = len(ts) * n * w.c
    return rows, 4 * w.head_dim * allowed


def cpu_baseline(w, arrays, min_seconds: float = 10.0):
    """The oracle as it stands, timed on a bounded sample of the same workload: R query
    rows of batch 0 spread evenly over the share, each as a full fp64 row against every
    key of the c blocks. R starts at 96 and doubles until one run of the oracle takes at
    least `min_seconds` (or covers the whole share); that run is reported."""
    import oracle
    from blockwise_ring_attention_amd.inputs import make_doc_start
    q, k, v = arrays
    ds = make_doc_start(w)
    total_rows = w.hq * w.rows
    count = 96
    while True:
        count = min(count, total_rows)
        rows, flop = cpu_sample(w, count)
        t0 = time.perf_counter()
        oracle.rank_forward(q, k, v, w.c, w.rank, w.causal, w.zigzag, rows=rows, doc_start=ds)
        sec = time.perf_counter() - t0
        if sec >= min_seconds or count == total_rows:
            break
        count *= 2
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
        "cpu_model": cpu_model(),
        "kind": "oracle",
        "sample": (f"{count} query rows of batch 0 spread evenly over the share of {w.name} (head-major), each "
                   f"a full fp64 row against all {w.c * w.rows} keys (masked entries computed and discarded); "
                   f"{sec:.1f} s wall; rate counts unmasked work only"),
        "seconds": sec,
        # every oracle row costs the same (a full row against every key), so the whole
        # share (all batches, heads and rows) scales linearly from the sample
        "full_share_seconds_estimate": round(sec * w.batch * total_rows / count, 1),
    }


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=3, help="untimed launches before the timed ones (at least)")
    ap.add_argument("--warmup-ms", type=float, default=WARMUP_MS,
                    help="the warmup also lasts at least this long: the graphics clock settles under load")
    ap.add_argument("--workload", default=DEFAULT_WORKLOAD)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle's CPU rate")
    ap.add_argument("--no-also", action="store_true", help="skip the other workloads timed beside the main one")
    ap.add_argument("--no-per-round", action="store_true",
                    help="skip the streamed form (one launch per ring round folding into a running "
                         "(out, lse), with an fp32 or bf16 running out, or plain launches plus ra_merge)")
    ap.add_argument("--balance", action="store_true",
                    help="only run the all-rank sweep (contiguous vs zigzag chunks) of the workload and print it")
    ap.add_argument("--sustain", type=float, default=0.0, metavar="SECONDS",
                    help="only run the workload back to back for SECONDS from idle and print the throughput "
                         "and the sampled clock and power over time")
    ap.add_argument("--timeline", type=int, default=0, metavar="LAUNCHES",
                    help="only run the workload through the diagnostic timeline build (built by the build "
                         "script) and print, for each of LAUNCHES recorded launches after the warmup, the "
                         "per-XCD finish times and stage times, and the per-tile prologue, tail and relaunch gap")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="minimum length of the timed oracle run for cpu_baseline")
    ap.add_argument("--lib", default=None, metavar="NAME_OR_PATH",
                    help="time another build of the library with the same C ABI: a design-choice ablation "
                         "name (xcd_scatter, no_swizzle, no_skip, one_head, stage_barrier, built by the build script) or a path")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="only run a plain device-to-device copy of MIB MiB three times (to scale the "
                         "FETCH_SIZE/WRITE_SIZE counters against a kernel of known traffic)")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one rank's share on one GPU; --gpus {args.gpus} is not supported "
              "(the library computes one rank's share; the ring's transfers between GPUs are not part of it)",
              file=sys.stderr)
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
    lib_used = None
    if args.lib:
        from blockwise_ring_attention_amd.csrc import build
        lib_used = args.lib if os.path.sep in args.lib else build.ablation_path(args.lib)
        _binding.use_library(lib_used)
    from blockwise_ring_attention_amd.inputs import make_inputs
    w = WORKLOADS[args.workload]
    if args.balance:
        sweep = balance_sweep(w, args.steps, args.warmup, args.warmup_ms)
        print(json.dumps({"balance_sweep": w.name, "c": w.c, "seq": w.seq, "steps": args.steps,
                          "warmup": args.warmup, **sweep}), flush=True)
        return
    if args.timeline:
        print(json.dumps({"timeline": w.name, **timeline_run(w, args.timeline, args.warmup_ms)}), flush=True)
        return
    flop, nbytes = workload_numbers(w)
    if args.sustain:
        print(json.dumps({"sustain": w.name, **sustain_run(w, args.sustain, flop)}), flush=True)
        return
    arrays = make_inputs(w)
    clock = ClockSampler()
    ms_step, ms_launch, ms_min, ms_med, warm_done = time_workload(w, args.steps, args.warmup, arrays, clock=clock,
                                                                 warmup_ms=args.warmup_ms)
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
        "warmup": warm_done,
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
                     "kernel_ms_min": round(ms_min, 4), "kernel_ms_median": round(ms_med, 4)},
    }
    line["kernel_sha"], line["library_sha"] = kernel_sha(), library_sha()
    if lib_used:
        line["library"] = os.path.relpath(lib_used, ROOT)
        line["roofline"]["traffic"] = None   # the committed counters describe the shipped kernel
    clk = clock.result()
    if "gfx_mhz_median" in clk:
        # the nominal peak assumes 2.4 GHz; at the clock held under this load it is lower
        clk["peak_at_observed_clock_tflops"] = round(peak * clk["gfx_mhz_median"] / 2400.0, 1)
        clk["frac_of_peak_at_observed_clock"] = round(achieved / clk["peak_at_observed_clock_tflops"], 4)
    line["clock"] = clk
    line["context"] = break_even_context(w, ms_launch, achieved)
    if not args.no_also:
        also = []
        for name in ALSO_WORKLOADS:
            wa = WORKLOADS[name]
            fa, _ = workload_numbers(wa)
            arrays_a = make_inputs(wa)
            clock_a = ClockSampler()
            ms_a, ml_a, _, _, steps_a, warm_a = time_workload_min(wa, args.steps, args.warmup, arrays_a,
                                                                   clock=clock_a, warmup_ms=args.warmup_ms)
            del arrays_a
            ca = clock_a.result()
            also.append({"workload": name, "value": round(fa / (ms_a * 1e-3) / 1e12, 2), "ms_per_step": round(ms_a, 4),
                         "kernel_ms_avg": round(ml_a, 4), "steps": steps_a, "warmup": warm_a,
                         "pct_of_peak": round(100 * fa / (ms_a * 1e-3) / 1e12 /
                                              (PEAK_BF16_TFLOPS if wa.dtype == "bf16" else PEAK_F32_TFLOPS), 2),
                         "peak_tflops": PEAK_BF16_TFLOPS if wa.dtype == "bf16" else PEAK_F32_TFLOPS,
                         "gfx_mhz_median": ca.get("gfx_mhz_median")})
        line["also"] = also
    if not args.no_per_round:
        what = {"accumulate": "one ra_rank_forward_accumulate launch per ring round (rounds [t, t+1)), each "
                              "folding its partial into an fp32 running (out, lse) in its epilogue; out rounded to "
                              "bf16 once at the end",
                "accumulate_bf16": "as accumulate with the running out kept in bf16 (round 0 a plain launch)",
                "merge": "one ra_rank_forward launch per ring round + in-place ra_merge into the running "
                         "(out, lse)",
                "accumulate_graph": "accumulate captured once in a HIP graph (the lse fill, the c launches and "
                                    "the final rounding) and replayed every step"}
        line["per_round"] = {}
        for mode in ("accumulate", "accumulate_bf16", "merge", "accumulate_graph"):
            ms_pr, round_ms, merge_ms, diff, lse_diff = time_per_round(w, max(1, args.steps // 4), 1, arrays, mode)
            line["per_round"][mode] = {
                "what": what[mode],
                "ms_per_step": round(ms_pr, 4), "value": round(flop / (ms_pr * 1e-3) / 1e12, 2),
                "overhead_vs_fused": round(ms_pr / ms_step - 1.0, 4),
                "round_kernel_ms": [round(x, 4) for x in round_ms], "merge_ms": [round(x, 4) for x in merge_ms],
                "max_abs_diff_vs_fused": diff, "lse_max_abs_diff_vs_fused": lse_diff}
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w, arrays, args.cpu_seconds)
    torch.cuda.synchronize()
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
