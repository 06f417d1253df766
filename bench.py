"""Throughput of the MoE re-routing operator (MoeReRoutingV2) on one MI355X.

A step is one whole call of the operator (offsets kernel + gather kernel) on
one batch of synthetic input already resident in HBM. The default workload is
the shape of the pages' single-operator example: A=16384 tokens of H=7168 int8
values, N=E=16, one huge segment, [A] fp32 scales (see
moe_token_re_amd/workloads.py for the recipe).

Calls rotate over several identical buffer sets whose total footprint is at
least 1 GiB, so the 256 MB Infinity Cache cannot hold the working set between
calls. Prints ONE JSON line:
  value       re-route GB/s = algorithmic bytes per call / wall time per call
  roofline    the dominant kernel alone (the fused kernel, or the gather
              kernel of the two-kernel path; the row map it reads is
              implementation traffic, not counted): algorithmic bytes per launch /
              its mean duration over back-to-back launches (HIP events on
              the launch stream) against 8 TB/s HBM;
              traffic from rocprofv3 FETCH_SIZE/WRITE_SIZE counters when the
              committed counter summary matches the current kernel source
  cpu_baseline the CPU oracle on the same workload, one host thread
plus the measured copy ceiling (hipMemcpyAsync device-to-device and a plain
16-byte non-temporal copy kernel moving the same token bytes), and the
per-call time of the same calls captured in one HIP graph and replayed
(us_per_call_graph: no host launch overhead, which matters for small calls;
the graph rotates over at most 1000 buffer sets, which for small calls fit
in the Infinity Cache).

With --inverse the same workload runs the inverse re-route (its token rows
taken as expert-major, returned to rank-major order), with the oracle's
inverse as the CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--inverse] [--no-cpu] [--no-ceiling]
"""
from __future__ import annotations

import argparse
import ctypes
import json
import math
import os
import re
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
METRIC = "re-route GB/s (bytes read+written) and % of HBM peak; µs/call A=16384 H=7168"
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "stream_gather_pages_shape_counters.txt")


def kernel_source_hash() -> str:
    """The hash of the library's current sources (the loaded library carries
    the same one, or loading it fails)."""
    from moe_token_re_amd import build

    return build.source_hash()


def bench_copy_lib():
    lib = ctypes.CDLL(os.path.join(ROOT, "moe_token_re_amd", "libmrr_bench_copy.so"))
    lib.mrr_bench_copy.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]
    lib.mrr_bench_copy.restype = ctypes.c_int
    lib.mrr_bench_device_facts.argtypes = [ctypes.c_int, ctypes.POINTER(ctypes.c_longlong)]
    lib.mrr_bench_device_facts.restype = ctypes.c_int
    return lib


def device_facts(torch, dev, lib) -> dict:
    """The device's compute units, LDS, clocks and caches, as HIP reports them."""
    props = torch.cuda.get_device_properties(dev)
    out = {"name": props.name, "arch": getattr(props, "gcnArchName", None), "hbm_bytes": props.total_memory}
    facts = (ctypes.c_longlong * 7)()
    if lib.mrr_bench_device_facts(dev.index or 0, facts) == 0:
        out.update({"compute_units": facts[0], "lds_bytes_per_cu": facts[1], "lds_bytes_per_workgroup_max": facts[2],
                    "shader_clock_mhz": facts[3] / 1000, "memory_clock_mhz": facts[4] / 1000,
                    "memory_bus_bits": facts[5], "l2_bytes": facts[6]})
    return out


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def gather_bytes_per_launch(w) -> int:
    """Algorithmic bytes of one gather launch: per row, the token row and the
    scale row read and written, the weight read and written, the index written."""
    per_row = 2 * w.token_row_bytes + 2 * w.scale_row_bytes + (8 if w.weight is not None else 0) + 4
    return per_row * w.A


def traffic_from_profile(w, kernel_name, direction="forward"):
    """HBM bytes per launch of the dominant kernel from the committed counter
    summary, scaled by the copy kernel's counter reading for a known byte
    count; None when the summary is missing, for another workload, kernel or
    direction, or the kernel source has changed since the counters were taken."""
    if not os.path.exists(PROFILE_SUMMARY):
        return None
    text = open(PROFILE_SUMMARY).read()
    fields = dict(re.findall(r"^(\w+):\s*(\S+)\s*$", text, flags=re.M))
    try:
        if (fields.get("source_hash") != kernel_source_hash() or fields.get("workload") != w.name
                or fields.get("kernel") != kernel_name or fields.get("direction", "forward") != direction):
            return None
        fetch = float(fields["FETCH_SIZE_KiB"]) * float(fields["fetch_scale"])
        write = float(fields["WRITE_SIZE_KiB"]) * float(fields["write_scale"])
    except (KeyError, ValueError):
        return None
    return int(round((fetch + write) * 1024))


def time_oracle(w, budget_s=3.0, max_runs=400, inverse=False):
    """The CPU oracle on the full workload, single-threaded, outputs preallocated
    and pre-faulted; median over runs that fit the time budget."""
    from oracle import oracle

    fn = oracle.reroute_inverse if inverse else oracle.reroute

    outs = oracle.allocate_outputs(w.tokens, w.counts, w.scales, w.weight)
    for o in outs:
        if o is not None:
            o.fill(0)
    times = []
    t_start = time.perf_counter()
    while len(times) < max_runs:
        t0 = time.perf_counter()
        fn(w.tokens, w.counts, w.scales, w.weight, w.etn_type, w.idx_type, out=outs)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s and len(times) >= 3:
            break
    return statistics.median(times), len(times)


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed calls (default 200; 1000 for the launch-bound tiny workload)")
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="pages_shape")
    ap.add_argument("--inverse", action="store_true", help="time the inverse re-route (expert-major -> rank-major)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU-oracle baseline")
    ap.add_argument("--no-ceiling", action="store_true", help="skip the copy-ceiling measurement")
    opt = ap.parse_args()
    if opt.steps is None:
        opt.steps = 1000 if opt.workload == "tiny" else 200

    if opt.gpus != 1:
        print(f"bench.py measures one GPU only (the operator is per-device and has no collectives); "
              f"--gpus {opt.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import numpy as np  # noqa: F401
    import torch

    from moe_token_re_amd import _lib, api, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.make(opt.workload)
    alg_bytes = w.algorithmic_bytes()
    bench_lib = bench_copy_lib()
    device = device_facts(torch, dev, bench_lib)
    print(f"[bench] device {device}", file=sys.stderr, flush=True)
    print(f"[bench] workload {w.name}: A={w.A} H={w.H} N={w.N} E={w.E} tokens={w.tokens_dtype} "
          f"algorithmic bytes/call={alg_bytes}", file=sys.stderr, flush=True)

    base = workloads.torch_inputs(w, dev)
    stream = torch.cuda.current_stream(dev)
    footprint = 2 * (w.A * (w.token_row_bytes + w.scale_row_bytes + 4 + (8 if w.weight is not None else 0)))
    n_sets = max(3, math.ceil((1 << 30) / max(footprint, 1)))
    calls = []
    inputs = []
    for k in range(n_sets):
        t = base if k == 0 else {key: (v.clone() if isinstance(v, torch.Tensor) else v) for key, v in base.items()}
        inputs.append(t)
        call, _ = api.make_call(t["tokens"], t["counts"], per_token_scales=t["scales"],
                                expert_topk_weight=t["weight"], expert_token_num_type=w.etn_type,
                                idx_type=w.idx_type, tokens_dtype=t["tokens_dtype"], stream=stream,
                                direction=_lib.INVERSE if opt.inverse else _lib.FORWARD)
        calls.append(call)
    torch.cuda.synchronize()

    # warmup
    for i in range(opt.warmup):
        calls[i % n_sets].run()
    torch.cuda.synchronize()
    for c in calls:
        c.run()
    torch.cuda.synchronize()
    st = calls[0].device_status()
    if st != _lib.SUCCESS:
        raise SystemExit(f"device status {_lib.status_string(st)}")

    # timed: exactly K whole calls, synchronized on both sides
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    ev0.record(stream)
    for i in range(opt.steps):
        calls[i % n_sets].run()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    ev_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall_s * 1e3 / opt.steps
    value = alg_bytes / (ms_per_step * 1e-3) / 1e9
    print(f"[bench] {opt.steps} calls: wall {ms_per_step * 1e3:.2f} us/call, events "
          f"{ev_ms * 1e3 / opt.steps:.2f} us/call, {value:.1f} GB/s", file=sys.stderr, flush=True)

    # the median of per-call event pairs (a separate pass: the events between
    # calls cost a little)
    pairs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(opt.steps)]
    torch.cuda.synchronize()
    for i, (a, b) in enumerate(pairs):
        a.record(stream)
        calls[i % n_sets].run()
        b.record(stream)
    torch.cuda.synchronize()
    per_call_median_us = statistics.median(a.elapsed_time(b) for a, b in pairs) * 1e3
    del pairs

    # per-kernel: K back-to-back launches of one kernel between two events on
    # the launch stream, rotating over the buffer sets. When the call is one
    # fused kernel that kernel is the dominant one; otherwise the gather
    # kernel is, timed on tables its sets' offsets kernels built beforehand.
    plan = calls[0].plan()
    n_k = max(opt.steps, 50)

    def back_to_back_us(fn):
        for i in range(min(10, n_k)):
            fn(calls[i % n_sets])
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(n_k):
            fn(calls[i % n_sets])
        ev1.record(stream)
        torch.cuda.synchronize()
        return ev0.elapsed_time(ev1) * 1e3 / n_k

    off_mean_us = None
    if plan["fused"]:
        kernel_name = "fused_kernel"
        kern_mean_us = back_to_back_us(lambda c: c.run())
        kbytes = alg_bytes
    else:
        kernel_name = "stream_gather_kernel" if plan["gather_kernel"] == 1 else "gather_kernel"
        off_mean_us = back_to_back_us(lambda c: c.run_offsets())
        for c in calls:
            c.run_offsets()
        kern_mean_us = back_to_back_us(lambda c: c.run_gather())
        kbytes = gather_bytes_per_launch(w)
    achieved = kbytes / (kern_mean_us * 1e-6) / 1e9
    print(f"[bench] plan {plan}", file=sys.stderr, flush=True)
    print(f"[bench] per kernel ({n_k} back-to-back launches): {kernel_name} {kern_mean_us:.2f} us, "
          f"{achieved:.1f} GB/s; offsets kernel {off_mean_us} us", file=sys.stderr, flush=True)

    # hot (same buffers every call), labelled as such
    torch.cuda.synchronize()
    ev0.record(stream)
    for _ in range(opt.steps):
        calls[0].run()
    ev1.record(stream)
    torch.cuda.synchronize()
    hot_us = ev0.elapsed_time(ev1) * 1e3 / opt.steps

    # the same calls captured in one HIP graph (the launch path allocates,
    # sets and synchronizes nothing) and replayed: the per-call cost without
    # the host's launch overhead, which dominates small calls
    side = torch.cuda.Stream(dev)
    n_cap = min(n_sets, 1000)  # calls per graph, each on its own buffer set
    gcalls = []
    for t in inputs[:n_cap]:
        gc, _ = api.make_call(t["tokens"], t["counts"], per_token_scales=t["scales"],
                              expert_topk_weight=t["weight"], expert_token_num_type=w.etn_type,
                              idx_type=w.idx_type, tokens_dtype=t["tokens_dtype"], stream=side,
                              direction=_lib.INVERSE if opt.inverse else _lib.FORWARD)
        gcalls.append(gc)
    with torch.cuda.stream(side):
        for gc in gcalls:
            gc.run()
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, stream=side):
        for i in range(n_cap):
            gcalls[i % len(gcalls)].run()
    torch.cuda.synchronize()
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, opt.steps // n_cap)
    t0 = time.perf_counter()
    for _ in range(reps):
        graph.replay()
    torch.cuda.synchronize()
    graph_us = (time.perf_counter() - t0) * 1e6 / (reps * n_cap)
    if any(gc.device_status() != _lib.SUCCESS for gc in gcalls[:1]):
        raise SystemExit("device status after graph replays")
    del graph, gcalls

    # copy ceiling over the same token bytes, same rotation
    ceiling = None
    if not opt.no_ceiling:
        nbytes16 = (w.A * w.token_row_bytes) // 16 * 16
        srcs = [c.args.tokens for c in calls]
        dsts = [torch.empty(nbytes16, dtype=torch.uint8, device=dev) for _ in range(n_sets)]
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_void_p]
        hip.hipMemcpyAsync.restype = ctypes.c_int
        hip_d2d = 3  # hipMemcpyDeviceToDevice
        s_ptr = stream.cuda_stream
        for i in range(10):
            assert bench_lib.mrr_bench_copy(dsts[i % n_sets].data_ptr(), srcs[i % n_sets], nbytes16, s_ptr) == 0
            assert hip.hipMemcpyAsync(dsts[i % n_sets].data_ptr(), srcs[i % n_sets], nbytes16, hip_d2d, s_ptr) == 0
        torch.cuda.synchronize()
        ev0.record(stream)
        for i in range(opt.steps):
            bench_lib.mrr_bench_copy(dsts[i % n_sets].data_ptr(), srcs[i % n_sets], nbytes16, s_ptr)
        ev1.record(stream)
        torch.cuda.synchronize()
        kern_us = ev0.elapsed_time(ev1) * 1e3 / opt.steps
        ev0.record(stream)
        for i in range(opt.steps):
            hip.hipMemcpyAsync(dsts[i % n_sets].data_ptr(), srcs[i % n_sets], nbytes16, hip_d2d, s_ptr)
        ev1.record(stream)
        torch.cuda.synchronize()
        memcpy_us = ev0.elapsed_time(ev1) * 1e3 / opt.steps
        ceil_gbps = max(2 * nbytes16 / (kern_us * 1e-6) / 1e9, 2 * nbytes16 / (memcpy_us * 1e-6) / 1e9)
        ceiling = {"copy_kernel_us": round(kern_us, 2), "memcpy_d2d_us": round(memcpy_us, 2),
                   "bytes_read_plus_written": 2 * nbytes16, "ceiling_GBps": round(ceil_gbps, 1),
                   "gather_frac_of_ceiling": round(achieved / ceil_gbps, 4),
                   "call_frac_of_ceiling": round(value / ceil_gbps, 4)}
        print(f"[bench] copy ceiling: kernel {kern_us:.2f} us, hipMemcpyAsync {memcpy_us:.2f} us, "
              f"{ceil_gbps:.1f} GB/s", file=sys.stderr, flush=True)
        del dsts

    cpu = None
    if not opt.no_cpu:
        med_s, runs = time_oracle(w, inverse=opt.inverse)
        cpu = {"value": round(alg_bytes / med_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"the full {w.name} workload (one whole call), median of {runs} runs, "
                         f"{med_s * 1e3:.1f} ms/call; host has {os.cpu_count()} logical CPUs",
               "cpu_model": cpu_model()}
        print(f"[bench] oracle: {med_s * 1e3:.1f} ms/call on 1 thread", file=sys.stderr, flush=True)

    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": opt.steps,
        "warmup": opt.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": w.name, "A": w.A, "H": w.H, "N": w.N, "E": w.E,
                   "tokens_dtype": w.tokens_dtype, "counts_dtype": str(w.counts.dtype),
                   "scales": None if w.scales is None else f"{w.scales_dtype}{list(w.scales.shape)}",
                   "topk_weight": w.weight is not None, "expert_token_num_type": w.etn_type,
                   "idx_type": w.idx_type, "direction": "inverse" if opt.inverse else "forward",
                   "buffer_sets": n_sets, "parallelism": "single GPU"},
        "us_per_call": round(ms_per_step * 1e3, 2),
        "us_per_call_events": round(ev_ms * 1e3 / opt.steps, 2),
        "us_per_call_event_pair_median": round(per_call_median_us, 2),
        "us_per_call_hot_same_buffers": round(hot_us, 2),
        "us_per_call_graph": round(graph_us, 2),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_call": alg_bytes,
        "launch_path": "fused single kernel" if plan["fused"] else "offsets kernel + gather kernel",
        "offsets_kernel_us_mean": None if off_mean_us is None else round(off_mean_us, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic_from_profile(w, kernel_name, "inverse" if opt.inverse else "forward"),
                     "kernel": kernel_name, "bytes_per_launch": kbytes,
                     "launch_us_mean": round(kern_mean_us, 2)},
        "copy_ceiling": ceiling,
        "cpu_baseline": cpu,
        "library_source_hash": _lib.library_source_hash(),
        "device": device,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
