"""Throughput of the MoE re-routing operator (MoeReRoutingV2) on one MI355X.

A step is one whole call of the operator (the one-launch stream kernel for
count matrices of at most 512 cells and token rows of 16-byte vectors from
32 bytes, the fused kernel for small calls, else offsets kernel + gather
kernel) on one batch of synthetic input already resident in HBM. The headline workload is the shape of the pages'
single-operator example: A=16384 tokens of H=7168 int8 values, N=E=16, one
huge segment, [A] fp32 scales (moe_token_re_amd/workloads.py has the recipe).

Calls rotate over several identical buffer sets whose total footprint is at
least 1 GiB, so the 256 MB Infinity Cache cannot hold the working set between
calls. Prints ONE JSON line:
  value        re-route GB/s = algorithmic bytes per call / wall time per call,
               the wall clock around exactly K calls, synchronized on both
               sides (nothing else inside the timed region)
  roofline     the dominant kernel alone (the one-launch kernel, the fused
               kernel, or the gather kernel of the two-kernel path):
               algorithmic bytes per launch / its
               mean duration, measured live as the mean period of K launches
               back to back between two HIP events on the launch stream (an
               event pair around each single launch adds ~2.5 us of its own).
               launch_us_rocprof is the average duration the committed
               rocprofv3 kernel-trace summary of this command holds for the
               same kernel (the profiler adds ~0.5 us per launch), given only
               when that summary was taken from the loaded library's sources.
               traffic: rocprofv3 FETCH_SIZE/WRITE_SIZE counters, under the
               same condition
  cpu_baseline the CPU oracle on the same workload, one host thread
  workloads    the other named workloads (and the inverse re-route at the
               pages' shape), each with its µs per call, GB/s, the gather's
               fraction of 8 TB/s and the call's and the gather's fractions of
               the measured copy ceiling (no oracle timing, no graph)
plus the measured copy ceiling (hipMemcpyAsync device-to-device and a plain
16-byte non-temporal copy kernel moving the same token bytes), and the
per-call time of the same calls captured in one HIP graph and replayed
(us_per_call_graph: no host launch overhead, which matters for small calls).

With --inverse the headline workload runs the inverse re-route (its token rows
taken as expert-major, returned to rank-major order), with the oracle's
inverse as the CPU baseline.

Usage: python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
                       [--inverse] [--no-cpu] [--no-ceiling] [--no-workloads]
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
PROFILE_SUMMARY = os.path.join(ROOT, "profiles", "stream_fused_pages_shape_counters.txt")
STATS_SUMMARY = os.path.join(ROOT, "profiles", "pages_shape_kernel_stats.md")
# the other workloads the default run reports (name, direction)
OTHER_WORKLOADS = (("tiny", "forward"), ("balanced_bf16", "forward"), ("mxfp8_skewed", "forward"),
                   ("tiny_segments", "forward"), ("pages_shape", "inverse"), ("odd_rows", "forward"),
                   ("experts_384", "forward"))


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


def rocprof_average_us(w, kernel_name, direction="forward"):
    """The committed rocprofv3 kernel-trace average duration (µs) of the kernel
    for this workload and direction; None unless the summary names them and
    was taken from the current sources."""
    if not os.path.exists(STATS_SUMMARY):
        return None
    fields = dict(re.findall(r"^(\w+):\s*(\S+)\s*$", open(STATS_SUMMARY).read(), flags=re.M))
    if (fields.get("source_hash") != kernel_source_hash() or fields.get("workload") != w.name
            or fields.get("direction", "forward") != direction):
        return None
    try:
        return float(fields[f"average_ns_{kernel_name}"]) / 1e3
    except (KeyError, ValueError):
        return None


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


class Bench:
    """One workload's calls on rotating buffer sets, and the timings of them."""

    def __init__(self, torch, dev, w, inverse, label):
        from moe_token_re_amd import _lib, api, workloads

        self.torch, self.dev, self.w, self.inverse, self.label = torch, dev, w, inverse, label
        self._lib = _lib
        self.stream = torch.cuda.current_stream(dev)
        base = workloads.torch_inputs(w, dev)
        footprint = 2 * (w.A * (w.token_row_bytes + w.scale_row_bytes + 4 + (8 if w.weight is not None else 0)))
        self.n_sets = max(3, math.ceil((1 << 30) / max(footprint, 1)))
        self.inputs, self.calls = [], []
        self.direction = _lib.INVERSE if inverse else _lib.FORWARD
        for k in range(self.n_sets):
            t = base if k == 0 else {key: (v.clone() if isinstance(v, torch.Tensor) else v) for key, v in base.items()}
            self.inputs.append(t)
            call, _ = api.make_call(t["tokens"], t["counts"], per_token_scales=t["scales"],
                                    expert_topk_weight=t["weight"], expert_token_num_type=w.etn_type,
                                    idx_type=w.idx_type, tokens_dtype=t["tokens_dtype"], stream=self.stream,
                                    direction=self.direction)
            self.calls.append(call)
        torch.cuda.synchronize()
        self.plan = self.calls[0].plan()
        self.alg_bytes = w.algorithmic_bytes()

    def warm(self, n):
        for i in range(n):
            self.calls[i % self.n_sets].run()
        for c in self.calls:
            c.run()
        self.torch.cuda.synchronize()
        st = self.calls[0].device_status()
        if st != self._lib.SUCCESS:
            raise SystemExit(f"{self.label}: device status {self._lib.status_string(st)}")

    def wall_us(self, k):
        """Wall time per call around exactly k whole calls, synchronized on
        both sides, with nothing else in the timed region."""
        torch, calls, n = self.torch, self.calls, self.n_sets
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(k):
            calls[i % n].run()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / k

    def _events(self, k):
        ev = self.torch.cuda.Event
        return [(ev(enable_timing=True), ev(enable_timing=True)) for _ in range(k)]

    def back_to_back_us(self, fn, k):
        """Mean period of k launches of fn between two events on the launch stream."""
        torch, calls, n, s = self.torch, self.calls, self.n_sets, self.stream
        for i in range(min(10, k)):
            fn(calls[i % n])
        torch.cuda.synchronize()
        e0, e1 = self._events(1)[0]
        e0.record(s)
        for i in range(k):
            fn(calls[i % n])
        e1.record(s)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / k

    def pair_us(self, fn, k):
        """Mean and median over k launches of fn of the span between an event
        recorded just before and one just after each launch."""
        torch, calls, n, s = self.torch, self.calls, self.n_sets, self.stream
        pairs = self._events(k)
        torch.cuda.synchronize()
        for i, (a, b) in enumerate(pairs):
            a.record(s)
            fn(calls[i % n])
            b.record(s)
        torch.cuda.synchronize()
        spans = [a.elapsed_time(b) * 1e3 for a, b in pairs]
        return statistics.mean(spans), statistics.median(spans)

    def kernel(self, k):
        """The dominant kernel: (name, algorithmic bytes per launch, back-to-back
        µs, event-pair mean µs), and the offsets kernel's back-to-back µs."""
        if self.plan["fused"]:
            run = lambda c: c.run()  # noqa: E731
            name = "stream_fused_kernel" if self.plan["fused"] == 2 else "fused_kernel"
            kbytes, off = self.alg_bytes, None
        else:
            name = "stream_gather_kernel" if self.plan["gather_kernel"] == 1 else "gather_kernel"
            kbytes = gather_bytes_per_launch(self.w)
            off = self.back_to_back_us(lambda c: c.run_offsets(), k)
            for c in self.calls:
                c.run_offsets()  # every set holds its row map for the gather-only launches
            run = lambda c: c.run_gather()  # noqa: E731
        b2b_us = self.back_to_back_us(run, k)
        pair_us, _ = self.pair_us(run, k)
        return name, kbytes, b2b_us, pair_us, off

    def copy_ceiling(self, lib, k):
        """The plain 16-byte streaming copy kernel and hipMemcpyAsync moving
        the workload's token bytes over the same rotation; the faster rate."""
        torch, w, n, s = self.torch, self.w, self.n_sets, self.stream
        nbytes16 = (w.A * w.token_row_bytes) // 16 * 16
        srcs = [c.args.tokens for c in self.calls]
        dsts = [torch.empty(nbytes16, dtype=torch.uint8, device=self.dev) for _ in range(n)]
        hip = ctypes.CDLL("libamdhip64.so")
        hip.hipMemcpyAsync.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t, ctypes.c_int,
                                       ctypes.c_void_p]
        hip.hipMemcpyAsync.restype = ctypes.c_int
        hip_d2d = 3  # hipMemcpyDeviceToDevice
        sp = s.cuda_stream
        for i in range(10):
            assert lib.mrr_bench_copy(dsts[i % n].data_ptr(), srcs[i % n], nbytes16, sp) == 0
            assert hip.hipMemcpyAsync(dsts[i % n].data_ptr(), srcs[i % n], nbytes16, hip_d2d, sp) == 0
        ev = torch.cuda.Event
        e0, e1 = ev(enable_timing=True), ev(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(s)
        for i in range(k):
            lib.mrr_bench_copy(dsts[i % n].data_ptr(), srcs[i % n], nbytes16, sp)
        e1.record(s)
        torch.cuda.synchronize()
        kern_us = e0.elapsed_time(e1) * 1e3 / k
        e0.record(s)
        for i in range(k):
            hip.hipMemcpyAsync(dsts[i % n].data_ptr(), srcs[i % n], nbytes16, hip_d2d, sp)
        e1.record(s)
        torch.cuda.synchronize()
        memcpy_us = e0.elapsed_time(e1) * 1e3 / k
        del dsts
        gbps = max(2 * nbytes16 / (kern_us * 1e-6) / 1e9, 2 * nbytes16 / (memcpy_us * 1e-6) / 1e9)
        return {"copy_kernel_us": round(kern_us, 2), "memcpy_d2d_us": round(memcpy_us, 2),
                "bytes_read_plus_written": 2 * nbytes16, "ceiling_GBps": round(gbps, 1)}

    def graph_us(self, k):
        """Per-call time of the same calls captured in one HIP graph (on a side
        stream, each call on its own buffer set, at most 1000) and replayed."""
        from moe_token_re_amd import api

        torch, w = self.torch, self.w
        side = torch.cuda.Stream(self.dev)
        n_cap = min(self.n_sets, 1000)
        gcalls = []
        for t in self.inputs[:n_cap]:
            gc, _ = api.make_call(t["tokens"], t["counts"], per_token_scales=t["scales"],
                                  expert_topk_weight=t["weight"], expert_token_num_type=w.etn_type,
                                  idx_type=w.idx_type, tokens_dtype=t["tokens_dtype"], stream=side,
                                  direction=self.direction)
            gcalls.append(gc)
        with torch.cuda.stream(side):
            for gc in gcalls:
                gc.run()
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph, stream=side):
            for gc in gcalls:
                gc.run()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        reps = max(1, k // n_cap)
        t0 = time.perf_counter()
        for _ in range(reps):
            graph.replay()
        torch.cuda.synchronize()
        us = (time.perf_counter() - t0) * 1e6 / (reps * n_cap)
        if gcalls[0].device_status() != self._lib.SUCCESS:
            raise SystemExit("device status after graph replays")
        return us


def launch_path(plan):
    return {2: "one-launch stream kernel", 1: "fused single kernel"}.get(plan["fused"],
                                                                         "offsets kernel + gather kernel")


def workload_summary(torch, dev, name, direction, copy_lib, steps):
    """µs per call, GB/s and roofline fractions of one more workload."""
    from moe_token_re_amd import workloads

    w = workloads.make(name)
    b = Bench(torch, dev, w, direction == "inverse", f"{name}/{direction}")
    k = 1000 if name == "tiny" else steps
    b.warm(10)
    us = b.wall_us(k)
    kname, kbytes, k_us, _, _ = b.kernel(k)
    ceil = b.copy_ceiling(copy_lib, k)
    gbps = b.alg_bytes / (us * 1e-6) / 1e9
    k_gbps = kbytes / (k_us * 1e-6) / 1e9
    out = {"direction": direction, "us_per_call": round(us, 2), "GBps": round(gbps, 1),
           "pct_hbm_peak": round(100 * gbps / HBM_PEAK_GBPS, 2), "algorithmic_bytes_per_call": b.alg_bytes,
           "path": launch_path(b.plan),
           "kernel": kname, "kernel_us_back_to_back": round(k_us, 2),
           "kernel_frac_of_8TBps": round(k_gbps / HBM_PEAK_GBPS, 4),
           "copy_ceiling_GBps": ceil["ceiling_GBps"],
           "kernel_frac_of_ceiling": round(k_gbps / ceil["ceiling_GBps"], 4),
           "call_frac_of_ceiling": round(gbps / ceil["ceiling_GBps"], 4), "calls_timed": k}
    print(f"[bench] {name}/{direction}: {out}", file=sys.stderr, flush=True)
    return out


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
    ap.add_argument("--no-workloads", action="store_true", help="skip the other workloads")
    opt = ap.parse_args()
    if opt.steps is None:
        opt.steps = 1000 if opt.workload == "tiny" else 200

    if opt.gpus != 1:
        print(f"bench.py measures one GPU only (the operator is per-device and has no collectives); "
              f"--gpus {opt.gpus} is not supported", file=sys.stderr)
        sys.exit(2)

    import torch

    from moe_token_re_amd import _lib, workloads

    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    w = workloads.make(opt.workload)
    copy_lib = bench_copy_lib()
    device = device_facts(torch, dev, copy_lib)
    print(f"[bench] device {device}", file=sys.stderr, flush=True)
    print(f"[bench] workload {w.name}: A={w.A} H={w.H} N={w.N} E={w.E} tokens={w.tokens_dtype} "
          f"algorithmic bytes/call={w.algorithmic_bytes()}", file=sys.stderr, flush=True)
    b = Bench(torch, dev, w, opt.inverse, w.name)
    b.warm(opt.warmup)

    # timed: exactly K whole calls, synchronized on both sides
    us = b.wall_us(opt.steps)
    value = b.alg_bytes / (us * 1e-6) / 1e9
    print(f"[bench] {opt.steps} calls: wall {us:.2f} us/call, {value:.1f} GB/s", file=sys.stderr, flush=True)

    # the same calls between two events (GPU time without the host's start and end)
    ev_us = b.back_to_back_us(lambda c: c.run(), opt.steps)
    _, pair_median_us = b.pair_us(lambda c: c.run(), opt.steps)
    n_k = max(opt.steps, 50)
    kname, kbytes, k_us, k_pair, off_us = b.kernel(n_k)
    achieved = kbytes / (k_us * 1e-6) / 1e9
    print(f"[bench] plan {b.plan}", file=sys.stderr, flush=True)
    print(f"[bench] {kname}: {k_us:.2f} us back to back, {achieved:.1f} GB/s ({k_pair:.2f} us per event pair); "
          f"offsets kernel {off_us} us back to back", file=sys.stderr, flush=True)

    # hot (same buffers every call), labelled as such
    b.torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(b.stream)
    for _ in range(opt.steps):
        b.calls[0].run()
    e1.record(b.stream)
    torch.cuda.synchronize()
    hot_us = e0.elapsed_time(e1) * 1e3 / opt.steps
    graph_us = b.graph_us(opt.steps)

    ceiling = None
    if not opt.no_ceiling:
        ceiling = b.copy_ceiling(copy_lib, opt.steps)
        ceiling["gather_frac_of_ceiling"] = round(achieved / ceiling["ceiling_GBps"], 4)
        ceiling["call_frac_of_ceiling"] = round(value / ceiling["ceiling_GBps"], 4)
        print(f"[bench] copy ceiling: {ceiling}", file=sys.stderr, flush=True)

    cpu = None
    if not opt.no_cpu:
        med_s, runs = time_oracle(w, inverse=opt.inverse)
        cpu = {"value": round(b.alg_bytes / med_s / 1e9, 3), "unit": "GB/s", "cores": 1, "kind": "oracle",
               "sample": f"the full {w.name} workload (one whole call), median of {runs} runs, "
                         f"{med_s * 1e3:.1f} ms/call; host has {os.cpu_count()} logical CPUs",
               "cpu_model": cpu_model()}
        print(f"[bench] oracle: {med_s * 1e3:.1f} ms/call on 1 thread", file=sys.stderr, flush=True)

    direction = "inverse" if opt.inverse else "forward"
    k_rp = rocprof_average_us(w, kname, direction)
    line = {
        "metric": METRIC,
        "value": round(value, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": opt.steps,
        "warmup": opt.warmup,
        "ms_per_step": round(us * 1e-3, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "u8",
        "data": "synthetic",
        "config": {"workload": w.name, "A": w.A, "H": w.H, "N": w.N, "E": w.E,
                   "tokens_dtype": w.tokens_dtype, "counts_dtype": str(w.counts.dtype),
                   "scales": None if w.scales is None else f"{w.scales_dtype}{list(w.scales.shape)}",
                   "topk_weight": w.weight is not None, "expert_token_num_type": w.etn_type,
                   "idx_type": w.idx_type, "direction": direction,
                   "buffer_sets": b.n_sets, "parallelism": "single GPU"},
        "us_per_call": round(us, 2),
        "us_per_call_events": round(ev_us, 2),
        "us_per_call_event_pair_median": round(pair_median_us, 2),
        "us_per_call_hot_same_buffers": round(hot_us, 2),
        "us_per_call_graph": round(graph_us, 2),
        "pct_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "algorithmic_bytes_per_call": b.alg_bytes,
        "launch_path": launch_path(b.plan),
        "offsets_kernel_us_back_to_back": None if off_us is None else round(off_us, 2),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(achieved / HBM_PEAK_GBPS, 4),
                     "traffic": traffic_from_profile(w, kname, direction),
                     "kernel": kname, "bytes_per_launch": kbytes,
                     "launch_us_mean": round(k_us, 2),
                     "launch_us_source": f"{n_k} launches back to back between two HIP events on the launch stream",
                     "launch_us_rocprof": None if k_rp is None else round(k_rp, 2),
                     "frac_rocprof": None if k_rp is None else round(kbytes / (k_rp * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
                     "launch_us_source_rocprof": None if k_rp is None else
                     "profiles/pages_shape_kernel_stats.md (rocprofv3 --kernel-trace --stats of this bench)"},
        "copy_ceiling": ceiling,
        "cpu_baseline": cpu,
        "library_source_hash": _lib.library_source_hash(),
        "device": device,
    }
    del b
    if not opt.no_workloads and not opt.inverse and w.name == "pages_shape":
        others = {}
        for name, d in OTHER_WORKLOADS:
            others[name if d == "forward" else f"{name}_{d}"] = workload_summary(
                torch, dev, name, d, copy_lib, max(50, min(opt.steps, 200)))
            torch.cuda.empty_cache()
        line["workloads"] = others
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
