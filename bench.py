#!/usr/bin/env python3
"""Allreduce throughput on one MI355X: essential GB/s and % of HBM peak.

A step is one in-place Allreduce of P rank buffers resident in HBM (one call of
ar_allreduce_ex), timed with HIP events on the stream it is launched on. Before
every step, outside the timed region, the inputs are restored from a pristine
copy (in-place sums grow the values) and the 256 MB Infinity Cache is flushed
by writing a 1 GiB buffer, so each step starts cold from HBM.

Essential bytes = P * n * elt read + P * n * elt written (every input read
once, every output written once). value = essential bytes / median time of the
call between two events (launch latency included); roofline.achieved =
essential bytes / mean device time of the call's kernel, from events the
library records around its own launch.

Default workload (the largest that fits one GPU): 7 ranks x 2^24 fp32
N(0, 1e-3), the generalized Allreduce over Z_7 with r = 0, fused replay; the
other schedules of that workload are reported beside it, and the 192-rank AHC
bf16 workload, the 10^4 x 106 fp32 small-message batches for P in {3, 6, 12, 24},
the 8-rank 2^20 fp32 workload and the 5-rank int32 workload follow under
"extra" (same method, fewer steps). Each schedule row carries the cost
reporter's step count and bytes and the fitted model's predicted time.

Other modes: --latency (graph-replayed single small calls), --model (fit
alpha/beta/gamma), --calibrate-copy (counter scaling), --summarize-profiles
(turn rocprofv3 output into the summaries under profiles/).
"""
from __future__ import annotations

import argparse
import csv
import glob
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure

# (algo, knob, exec[, collective[, op[, steps[, factors]]]])
WORKLOADS = {
    "prime_fp32": dict(
        desc="7 ranks x 2^24 fp32 N(0,1e-3), seed 0",
        P=7, n=1 << 24, dtype="fp32", batch=1, groups=None,
        headline=("generalized", 0, "fused"),
        others=[("direct", 0, "fused"), ("ring", 0, "fused"), ("rh_rd", 0, "fused"),
                ("generalized", 1, "fused"), ("generalized", 2, "fused"), ("generalized", 3, "fused"),
                ("generalized", 1, "dag"), ("generalized", 2, "dag"), ("generalized", 3, "dag"),
                ("generalized", 0, "fused", "allreduce", "sum", 4), ("generalized", 0, "fused", "allreduce", "sum", 5),
                ("generalized", 0, "fused", "allreduce", "sum", 6),
                ("rd", 0, "fused"), ("binomial", 0, "fused"), ("chain", 1, "fused"),
                ("generalized", 0, "fused", "allreduce", "avg"), ("generalized", 0, "fused", "allreduce", "max"),
                ("generalized", 0, "fused", "reduce_scatter"), ("ring", 0, "fused", "reduce_scatter"),
                ("generalized", 0, "fused", "all_gather"), ("ring", 0, "fused", "all_gather"),
                ("generalized", 0, "literal"), ("generalized", 3, "literal"), ("ring", 0, "literal"),
                ("rh_rd", 0, "literal"), ("generalized", 0, "literal", "allreduce", "sum", 6),
                ("chain", 8, "literal")]),
    "ahc_bf16": dict(
        desc="192 ranks in groups (64, 128) x 2^20 bf16 N(0,1), fp32 accumulation, seed 0",
        P=192, n=1 << 20, dtype="bf16", batch=1, groups=[64, 128],
        headline=("ahc", 0, "fused"),
        others=[("ahc", 0, "fused", "allreduce", "max"), ("direct", 0, "fused"), ("ring", 0, "fused"),
                ("rh_rd", 0, "fused"), ("generalized", 0, "fused"), ("ahc", 0, "fused", "allreduce", "avg"),
                ("ahc", 0, "literal")]),
    "small_batch": dict(
        desc="P ranks x 10^4 instances x 106 fp32 U(-1,1), seed 0",
        P=24, n=106, dtype="fp32", batch=10_000, groups=None, steps=100,
        headline=("rd", 0, "fused"),
        others=[("binomial", 0, "fused"), ("direct", 0, "fused"), ("generalized", "L", "fused"),
                ("generalized", "L", "dag"), ("generalized", 0, "fused"), ("ring", 0, "fused"),
                ("rd", 0, "literal"), ("binomial", 0, "literal"), ("generalized", "L", "literal")]),
    "rh_fp32": dict(
        desc="8 ranks x 2^20 fp32 N(0,1), seed 0",
        P=8, n=1 << 20, dtype="fp32", batch=1, groups=None, warm=True,
        headline=("rh_rd", 0, "fused"),
        others=[("ring", 0, "fused"), ("direct", 0, "fused"), ("rd", 0, "fused"), ("generalized_xor", 0, "fused"),
                ("generalized", 0, "fused"), ("rh_rd", 0, "literal"), ("ring", 0, "literal")]),
    "ring_int32": dict(
        desc="5 ranks x 4096 int32 U[-2^20, 2^20], seed 0",
        P=5, n=4096, dtype="int32", batch=1, groups=None, steps=100,
        headline=("ring", 0, "fused"),
        others=[("direct", 0, "fused"), ("ring", 0, "literal")]),
}
SMALL_BATCH_P = (3, 6, 12, 24)
# the workloads the default run reports under "extra" (small_batch once per P)
EXTRA_WORKLOADS = ("ahc_bf16", "small_batch", "rh_fp32", "ring_int32")

DT_NAME = {"fp32": "f32", "bf16": "bf16", "int32": "i32"}
ELT = {"fp32": 4, "bf16": 2, "int32": 4}


def ceil_log2(P: int) -> int:
    return (P - 1).bit_length()


def kernel_source_hash() -> str:
    """Hash of the device code and of the executor that lays out its work items."""
    h = hashlib.sha256()
    for name in ("kernels.h", "launch.h", "exec.hip", "jit.cpp"):
        with open(os.path.join(ROOT, "allreduce_schedule_algorithms_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def workload(name: str, P: int | None = None) -> dict:
    wl = dict(WORKLOADS[name])
    wl["name"] = name
    if name == "small_batch" and P is not None:
        wl["P"] = P
    wl["entries"] = [resolve_entry(wl, e) for e in [wl["headline"]] + wl["others"]]
    return wl


def workload_label(wl) -> str:
    desc = wl["desc"].replace("P ranks", "%d ranks" % wl["P"])
    return "%s: %s" % (wl["name"], desc)


def resolve_entry(wl, e):
    """Knob "L" stands for ceil(log2 P) (the latency-optimal generalized version)."""
    e = list(e)
    if e[1] == "L":
        e[1] = ceil_log2(wl["P"])
    return tuple(e)


def make_inputs(wl):
    from synth import inputs
    if wl["name"] == "small_batch":
        return inputs.workload("small_batch", P=wl["P"])
    return inputs.workload(wl["name"])


def host_to_device(x, dtype):
    import numpy as np
    import torch
    if dtype == "bf16":
        t = torch.from_numpy(np.ascontiguousarray(x).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(x))
    return t.cuda()


def essential_bytes(wl, coll="allreduce"):
    """Every input read once, every output written once: 2 P n (Allreduce),
    P n + n (reduce-scatter: one part out per rank), P n (all-gather: each part
    read at its owner and written to the P - 1 others)."""
    pn = float(wl["P"]) * wl["n"] * wl["batch"] * ELT[wl["dtype"]]
    n1 = float(wl["n"]) * wl["batch"] * ELT[wl["dtype"]]
    return {"allreduce": 2.0 * pn, "reduce_scatter": pn + n1, "all_gather": pn}[coll]


class KernelEvents:
    """Raw HIP timing events created with hipEventDisableSystemFence, for the
    library's ar_call.start_event / stop_event. torch.cuda.Event has no such
    flag; its default events add a system-scope release when the stop event is
    recorded (about 2 us on a 13 us kernel), which a kernel's device time does
    not include and rocprofv3's kernel trace does not show."""
    DISABLE_SYSTEM_FENCE = 0x20000000

    def __init__(self):
        import ctypes as C

        import torch  # noqa: F401  (loads the HIP runtime the library shares)
        path = None
        with open("/proc/self/maps") as f:
            for line in f:
                if "libamdhip64" in line:
                    path = line.split()[-1]
                    break
        self.C = C
        self.hip = C.CDLL(path or "libamdhip64.so")
        self.hip.hipEventCreateWithFlags.argtypes = [C.POINTER(C.c_void_p), C.c_uint]
        self.hip.hipEventElapsedTime.argtypes = [C.POINTER(C.c_float), C.c_void_p, C.c_void_p]
        self.hip.hipEventDestroy.argtypes = [C.c_void_p]

    def create(self):
        e = self.C.c_void_p()
        rc = self.hip.hipEventCreateWithFlags(self.C.byref(e), self.DISABLE_SYSTEM_FENCE)
        if rc != 0:
            raise RuntimeError(f"hipEventCreateWithFlags failed ({rc})")
        return e.value

    def elapsed_ms(self, a, b):
        f = self.C.c_float()
        rc = self.hip.hipEventElapsedTime(self.C.byref(f), a, b)
        if rc != 0:
            raise RuntimeError(f"hipEventElapsedTime failed ({rc})")
        return f.value

    def destroy(self, evs):
        for a, b in evs:
            self.hip.hipEventDestroy(a)
            self.hip.hipEventDestroy(b)


class Runner:
    def __init__(self, wl, x, flush):
        import torch

        import allreduce_schedule_algorithms_amd as A
        self.A = A
        self.wl = wl
        self.stream = torch.cuda.Stream()
        self.pristine = host_to_device(x, wl["dtype"])           # (P, batch*n)
        self.work = torch.empty_like(self.pristine)
        self.flush = flush
        self.ptrs = [self.work[p].data_ptr() for p in range(wl["P"])]
        self.kernel_events = KernelEvents()

    def call_for(self, algo, knob, ex, start_event=None, stop_event=None, coll="allreduce", op="sum", rsteps=0,
                 factors=None):
        wl = self.wl
        return self.A.make_call(wl["P"], wl["n"], wl["dtype"], op, algo, knob, ex, wl["batch"],
                                wl["groups"] if algo == "ahc" else factors,
                                start_event=start_event, stop_event=stop_event, collective=coll, steps=rsteps)

    def prep(self, cold=True):
        import torch
        with torch.cuda.stream(self.stream):
            self.work.copy_(self.pristine)
            if cold:
                self.flush.zero_()

    def time(self, algo, knob, ex, steps, warmup, cold=True, kernel_pass=True, coll="allreduce", op="sum",
             rsteps=0, factors=None):
        """Per step: (untimed) restore + flush, then the timed call.

        Pass 1 brackets each plain call with two events on the library's stream
        (what a caller waits for, launch latency included): value, ms_per_step.
        Pass 2 repeats the steps with ar_call.start_event / stop_event, which the
        library records at the start and end of its own kernels: the kernels'
        device time, the figure rocprofv3's kernel trace reports. These events
        carry no system-scope fence (KernelEvents).
        """
        import torch
        st = self.stream

        def ev():
            e = torch.cuda.Event(enable_timing=True)
            e.record(st)  # creates the underlying hipEvent_t
            return e

        plain = self.call_for(algo, knob, ex, coll=coll, op=op, rsteps=rsteps, factors=factors)
        essential = essential_bytes(self.wl, coll)
        for _ in range(warmup):
            self.prep(cold)
            self.A.ar_allreduce_ex(self.ptrs, plain, st)
        call_evs = [(ev(), ev()) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            self.prep(cold)
            call_evs[k][0].record(st)
            self.A.ar_allreduce_ex(self.ptrs, plain, st)
            call_evs[k][1].record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [a.elapsed_time(b) for a, b in call_evs]
        med = statistics.median(ms)
        out = dict(ms=med, ms_mean=statistics.fmean(ms), ms_min=min(ms), wall_ms_per_step=1e3 * wall / steps,
                   GBps=essential / (med * 1e-3) / 1e9)
        if kernel_pass:
            kev = self.kernel_events
            kern_evs = [(kev.create(), kev.create()) for _ in range(steps)]
            calls = [self.call_for(algo, knob, ex, a, b, coll, op, rsteps, factors) for a, b in kern_evs]
            torch.cuda.synchronize()
            for k in range(steps):
                self.prep(cold)
                self.A.ar_allreduce_ex(self.ptrs, calls[k], st)
            torch.cuda.synchronize()
            kms = [kev.elapsed_ms(a, b) for a, b in kern_evs]
            kev.destroy(kern_evs)
            kmean = statistics.fmean(kms)
            out.update(kernel_ms=kmean, kernel_ms_median=statistics.median(kms),
                       kernel_GBps=essential / (kmean * 1e-3) / 1e9)
        return out

    def unbatched(self, algo, knob, calls):
        """``calls`` separate one-instance Allreduces (instance b at offset b * n
        of every rank's buffer), back to back on one stream: the per-call time
        is the library's per-call alpha on this device (host + launch +
        kernel)."""
        import torch
        wl = self.wl
        st = self.stream
        elt = ELT[wl["dtype"]]
        call = self.A.make_call(wl["P"], wl["n"], wl["dtype"], "sum", algo, knob, "fused", 1, None)
        calls = min(calls, wl["batch"])
        ptr_sets = [self.A.marshal_ptrs([p + b * wl["n"] * elt for p in self.ptrs]) for b in range(calls)]
        self.prep(cold=False)
        for b in range(min(calls, 50)):  # warm: plans built, caches filled
            self.A.ar_allreduce_ex(ptr_sets[b], call, st)
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        a.record(st)
        for b in range(calls):
            self.A.ar_allreduce_ex(ptr_sets[b], call, st)
        z.record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        out = {"calls": calls, "us_per_call": round(a.elapsed_time(z) * 1e3 / calls, 3),
               "wall_us_per_call": round(wall * 1e6 / calls, 3), "schedule": f"{algo}/r{knob}/fused",
               "kernel": KERNEL_NAMES[self.A.ar_kernel_of(call).name]}
        # the same calls captured once in a HIP graph and replayed: the device's
        # per-call time without the host's enqueue cost (plans are built above)
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for b in range(calls):
                self.A.ar_allreduce_ex(ptr_sets[b], call, st)
        g.replay()
        torch.cuda.synchronize()
        with torch.cuda.stream(st):
            a.record(st)
            g.replay()
            z.record(st)
        torch.cuda.synchronize()
        out["graph_us_per_call"] = round(a.elapsed_time(z) * 1e3 / calls, 3)
        del g
        return out

    def ceiling(self, reps=10):
        """Cold-HBM bandwidth of the probe kernels (libar_probe.so) on this
        workload's buffers: the 2P in-place streams of the direct kernel's
        access pattern (P reads + P writes per element offset), and one plain
        copy of the same total bytes (1 read + 1 write stream). Best of 1, 2 and
        4 vectors per thread, median of `reps` flushed launches each."""
        import torch

        from allreduce_schedule_algorithms_amd import probe
        wl = self.wl
        nbytes = wl["n"] * wl["batch"] * ELT[wl["dtype"]] // 16 * 16
        P = wl["P"]
        kev = self.kernel_events
        st = self.stream
        total = 2.0 * P * nbytes
        flat = self.work.view(-1)
        half = flat.numel() // 2 * flat.element_size() // 16 * 16
        out = {}
        kinds = [(probe.AR_PROBE_STREAMS, "streams_2P", self.ptrs, total),
                 (probe.AR_PROBE_COPY, "copy_1r1w", [flat.data_ptr(), flat.data_ptr() + half], 2.0 * half)]
        if P in (7, 8) and wl["dtype"] == "fp32":
            kinds.append((probe.AR_PROBE_FOLD, "fold_2P", self.ptrs, total))
        for kind, name, ptrs, moved in kinds:
            per_m = {}
            for m in (1, 2, 4):
                evs = [(kev.create(), kev.create()) for _ in range(reps + 2)]
                nb = half if kind == probe.AR_PROBE_COPY else nbytes
                for a, b in evs:
                    self.prep(cold=True)
                    probe.ar_probe_stream(ptrs, nb, kind, m, st, a, b)
                torch.cuda.synchronize()
                ms = statistics.median([kev.elapsed_ms(a, b) for a, b in evs[2:]])
                kev.destroy(evs)
                per_m[m] = round(moved / (ms * 1e-3) / 1e9, 1)
            best = max(per_m, key=per_m.get)
            out[name] = {"GBps": per_m[best], "vectors_per_thread": best, "by_vectors": per_m,
                         "bytes": moved}
        out["best_2P"] = max(v["GBps"] for k, v in out.items() if k.endswith("_2P"))
        out["note"] = ("probe kernels (libar_probe.so), cold Infinity Cache, kernel device time: streams_2P "
                       "reads and writes back every rank buffer in place as the direct kernel's access "
                       "pattern does; fold_2P is the smallest one-pass Allreduce kernel (fp32 sum compiled for "
                       "P, no work items, no rank table); copy_1r1w copies half the workload's bytes to the "
                       "other half; best_2P is the faster of the two 2P-stream kernels")
        return out


def cpu_baseline(wl, x, budget_s=12.0):
    """The oracle, as it stands, on this host: repeated replays of the headline schedule."""
    import numpy as np

    import oracle
    algo, knob, _ = wl["entries"][0][:3]
    P, n, B = wl["P"], wl["n"], wl["batch"]
    if B > 1:
        xs = x.reshape(P, B, n)
        sample = f"full workload ({B} instances of {n})"
        ess = 2.0 * P * n * B * ELT[wl["dtype"]]
        idx = None
    elif P * n > (1 << 24):
        # bounded sample: about 2^24 values in all, evenly spaced offsets
        idx = np.unique(np.linspace(0, n - 1, num=min(n, (1 << 24) // P), dtype=np.int64))
        xs = np.ascontiguousarray(x[:, idx])
        sample = f"{len(idx)} of {n} offsets per rank (evenly spaced, all parts covered)"
        ess = 2.0 * P * len(idx) * ELT[wl["dtype"]]
    else:
        xs = x
        idx = None
        sample = f"full workload ({P} x {n})"
        ess = 2.0 * P * n * ELT[wl["dtype"]]
    times = []
    t_start = time.perf_counter()
    while True:
        t0 = time.perf_counter()
        if idx is None:
            oracle.allreduce(xs, algo, wl["dtype"], "sum", knob=knob, groups=wl["groups"],
                             n=n if B > 1 else None)
        else:
            oracle.allreduce(xs, algo, wl["dtype"], "sum", knob=knob, groups=wl["groups"], n=n, idx=idx)
        times.append(time.perf_counter() - t0)
        if time.perf_counter() - t_start > budget_s or len(times) >= 50:
            break
    mean = statistics.fmean(times)
    return {"value": round(ess / mean / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{sample}; {algo} r={knob} replay, {len(times)} runs, mean {mean:.3f} s (NumPy, one "
                      f"thread); host {host_cpu()}",
            "brute_force": brute_force_all_cores(xs, wl["dtype"])}


def host_cpu():
    model = "unknown CPU"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return f"{model}, {os.cpu_count()} logical CPUs"


def brute_force_all_cores(xs, dtype, budget_s=4.0):
    """The plain elementwise reduction of all ranks (no schedule), in threads
    over element ranges; NumPy releases the GIL in the adds. Same sample as the
    oracle leg; bf16 is widened to fp32 first, int32 sums wrap."""
    import concurrent.futures as cf

    import numpy as np
    x = np.asarray(xs)
    P = x.shape[0]
    flat = x.reshape(P, -1)
    if dtype == "bf16":
        flat = (flat.astype(np.uint32) << 16).view(np.float32)
    elif dtype == "int32":
        flat = flat.view(np.uint32)
    m = flat.shape[1]
    threads = max(1, min(16, os.cpu_count() or 1))
    cuts = np.linspace(0, m, threads + 1).astype(np.int64)

    def part(i):
        lo, hi = cuts[i], cuts[i + 1]
        acc = flat[0, lo:hi].copy()
        for p in range(1, P):
            acc += flat[p, lo:hi]
        return acc

    times = []
    t_start = time.perf_counter()
    with cf.ThreadPoolExecutor(threads) as ex:
        while True:
            t0 = time.perf_counter()
            list(ex.map(part, range(threads)))
            times.append(time.perf_counter() - t0)
            if time.perf_counter() - t_start > budget_s or len(times) >= 20:
                break
    mean = statistics.fmean(times)
    ess = 2.0 * x.size * x.dtype.itemsize  # read every input, write one result per rank
    return {"value": round(ess / mean / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "brute-force elementwise reduction (no schedule)"}


LATENCY_CASES = [  # (P, n, algo, knob): one 106-fp32 instance (about 425 bytes) per rank, and neighbours
    (2, 106, "direct", 0), (8, 106, "direct", 0), (24, 106, "direct", 0), (24, 1, "direct", 0),
    (3, 106, "rd", 0), (6, 106, "rd", 0), (12, 106, "rd", 0), (24, 106, "rd", 0), (24, 106, "binomial", 0),
    (24, 106, "generalized", 5), (8, 106, "rh_rd", 0), (8, 106, "ring", 0),
    (127, 106, "generalized", 0), (127, 106, "generalized", 4), (127, 106, "generalized", 7),
]


def latency(calls=2000):
    """Per-call device time of single small Allreduces: `calls` calls on
    consecutive instances, captured once in a HIP graph and replayed, timed
    with events around the replay. Without the host's enqueue cost this is the
    library's alpha on this device (launch, one kernel, completion). Literal
    execution of the same call (one launch per step) and the DAG replay
    (AR_EXEC_DAG) are timed the same way."""
    import numpy as np
    import torch

    import allreduce_schedule_algorithms_amd as A
    from synth import inputs
    rows = []
    for P, n, algo, knob in LATENCY_CASES:
        reps = calls if P <= 32 else calls // 10
        x = inputs.make("fp32", P, n * reps, seed=1)
        bufs = [torch.from_numpy(np.ascontiguousarray(x[p])).cuda() for p in range(P)]
        st = torch.cuda.Stream()
        ptrs = [A.marshal_ptrs([b.data_ptr() + i * n * 4 for b in bufs]) for i in range(reps)]
        row = {"P": P, "n": n, "schedule": f"{algo}/r{knob}"}
        for ex in ("fused", "dag", "literal"):
            call = A.make_call(P, n, "fp32", "sum", algo, knob, ex)
            with torch.cuda.stream(st):
                for i in range(20):  # plans and workspace built outside the capture
                    A.ar_allreduce_ex(ptrs[i], call, st)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g, stream=st):
                for i in range(reps):
                    A.ar_allreduce_ex(ptrs[i], call, st)
            g.replay()
            torch.cuda.synchronize()
            a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            with torch.cuda.stream(st):
                a.record(st)
                g.replay()
                z.record(st)
            torch.cuda.synchronize()
            row[f"{ex}_kernel"] = KERNEL_NAMES[A.ar_kernel_of(call).name]
            row[f"{ex}_us_per_call"] = round(a.elapsed_time(z) * 1e3 / reps, 3)
            del g
        rows.append(row)
        print(json.dumps(row), file=sys.stderr, flush=True)
        del bufs
    return {"latency_fp32_graph_replay": rows, "calls": calls}


def model_fit(args):
    """Fit the alpha-beta-gamma model to this device and check its choices.

    Literal execution runs one launch per schedule step, so a call costs about
    alpha per step plus beta per byte moved and gamma per byte combined -- the
    generalized-Allreduce paper's model, whose parameters the paper measured on
    its cluster before choosing r. Here every rank is a buffer in one HBM, so the
    natural byte counts are the sums over ranks ("all_ranks"); the paper's
    per-link form ("busiest": per step the busiest rank) is fitted too for
    comparison. Both fits are relative least squares over every schedule at
    P = 7 and 8 and sizes 2^10..2^22; P = 127 at 2^8..2^16 elements (the paper's
    small-message experiment) is held out: there the fitted model's choice of r
    is compared with the measured fastest r, and the time lost by following the
    model is reported. A model-only table of the generalized algorithm's best
    time over the best of recursive doubling, recursive halving + doubling and
    ring (the paper's Fig. 1 ratio) closes the output."""
    import numpy as np
    import torch

    import allreduce_schedule_algorithms_amd as A
    from synth import inputs

    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")
    st = torch.cuda.Stream()

    def timed(P, n, algo, knob, reps=12):
        x = inputs.make("fp32", P, n, seed=1)
        pristine = torch.from_numpy(x).cuda()
        work = torch.empty_like(pristine)
        ptrs = [work[p].data_ptr() for p in range(P)]
        call = A.make_call(P, n, "fp32", "sum", algo, knob, "literal")
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(reps)]
        for k in range(reps + 2):
            with torch.cuda.stream(st):
                work.copy_(pristine)
                flush.zero_()
            if k >= 2:
                evs[k - 2][0].record(st)
            A.ar_allreduce_ex(ptrs, call, st)
            if k >= 2:
                evs[k - 2][1].record(st)
        torch.cuda.synchronize()
        return statistics.median([a.elapsed_time(b) for a, b in evs]) * 1e-3

    def features(P, n, algo, knob):
        s = A.ar_schedule_build(A.make_call(P, n, "fp32", "sum", algo, knob, "literal"))
        sent, recv, red = s.cost_steps(P)
        steps = sent.shape[0]
        busiest_b = float(np.maximum(sent, recv).max(axis=1).sum()) * 4 if steps else 0.0
        busiest_g = float(red.max(axis=1).sum()) * 4 if steps else 0.0
        return dict(steps=steps, all_ranks_b=float(sent.sum()) * 4, all_ranks_g=float(red.sum()) * 4,
                    busiest_b=busiest_b, busiest_g=busiest_g)

    def cands(P):
        L = (P - 1).bit_length()
        return [("direct", 0), ("ring", 0), ("rh_rd", 0), ("rd", 0), ("binomial", 0)] + \
            [("generalized", r) for r in range(L + 1)]

    def run(Ps, sizes):
        rows = []
        for P in Ps:
            for n in sizes:
                for algo, knob in cands(P):
                    row = dict(P=P, n=n, algo=algo, knob=knob, **features(P, n, algo, knob))
                    row["seconds"] = timed(P, n, algo, knob)
                    rows.append(row)
                print(f"model: P={P} n={n} done", file=sys.stderr, flush=True)
        return rows

    fit_rows = run((7, 8), (1 << 10, 1 << 14, 1 << 17, 1 << 20, 1 << 22))
    held_rows = run((127,), (1 << 8, 1 << 10, 1 << 12, 1 << 14, 1 << 16))

    def fit(form):
        X = np.array([[r["steps"], r[form + "_b"], r[form + "_g"]] for r in fit_rows])
        y = np.array([r["seconds"] for r in fit_rows])
        w = 1.0 / y  # relative least squares: every case counts alike
        from scipy.optimize import nnls
        coef, _ = nnls(X * w[:, None], y * w)  # non-negative parameters
        rel = np.abs(X @ coef - y) / y
        return coef, rel

    def pred(row, coef, form):
        return coef[0] * row["steps"] + coef[1] * row[form + "_b"] + coef[2] * row[form + "_g"]

    out = {"fits": {}, "held_out_P127": {}}
    for form in ("all_ranks", "busiest"):
        coef, rel = fit(form)
        held_rel = [abs(pred(r, coef, form) - r["seconds"]) / r["seconds"] for r in held_rows]
        choice = []
        for n in sorted({r["n"] for r in held_rows}):
            gen = [r for r in held_rows if r["n"] == n and r["algo"] == "generalized"]
            meas = min(gen, key=lambda r: r["seconds"])
            mod = min(gen, key=lambda r: (pred(r, coef, form), r["steps"]))
            choice.append(dict(n=n, measured_best_r=meas["knob"], model_best_r=mod["knob"],
                               loss_vs_best=round(mod["seconds"] / meas["seconds"] - 1, 4),
                               times_us={r["knob"]: round(r["seconds"] * 1e6, 1) for r in gen}))
        out["fits"][form] = dict(alpha_s=float(coef[0]), beta_s_per_byte=float(coef[1]),
                                 gamma_s_per_byte=float(coef[2]), median_rel_error=float(np.median(rel)),
                                 max_rel_error=float(np.max(rel)),
                                 held_out_median_rel_error=float(np.median(held_rel)))
        out["held_out_P127"][form] = choice
    # the paper's Fig. 1 quantity (host only), with the all-ranks fit's alpha,
    # beta, gamma in both forms: "busiest" prices them as if every rank had its
    # own memory path, "all_ranks" as this device does
    coef = [out["fits"]["all_ranks"][k] for k in ("alpha_s", "beta_s_per_byte", "gamma_s_per_byte")]
    for form in ("busiest", "all_ranks"):
        A.ar_set_cost_model(*coef, form)
        grid = []
        try:
            for P in (5, 7, 12, 24, 63, 100, 127):
                for n in (1 << 6, 1 << 10, 1 << 14, 1 << 18, 1 << 22):
                    def t(algo, knob=0):
                        return A.ar_select(A.make_call(P, n, "fp32", "sum", algo, knob, "literal"))[2]
                    best_sota = min(t("rd"), t("rh_rd"), t("ring"))
                    a, r, tg = A.ar_select(A.make_call(P, n, "fp32", "sum", "generalized", -1, "literal"))
                    grid.append(dict(P=P, n=n, r=r, ratio=round(tg / best_sota, 4)))
        finally:
            A.ar_set_cost_model()
        out["fig1_ratio_" + form] = grid
    out["cases"] = dict(fit=len(fit_rows), held_out=len(held_rows))
    out["rows"] = fit_rows + held_rows
    print(json.dumps(out))


def schedule_key(algo, knob, ex, coll="allreduce", op="sum", rsteps=0, factors=None):
    """Key of a schedule in the bench's table: algo/r<knob>/<exec>[/<collective>][/<op>][/S<steps>][/Z<factors>]."""
    key = f"{algo}/r{knob}/{ex}" + ("" if coll == "allreduce" else f"/{coll}") + ("" if op == "sum" else f"/{op}")
    key += f"/S{rsteps}" if rsteps else ""
    key += "/Z" + "x".join(str(m) for m in factors) if factors else ""
    return key


def parse_key(key):
    algo, k, ex, *rest = key.split("/")
    return dict(algo=algo, knob=int(k[1:]), ex=ex,
                coll=next((t for t in rest if t in ("reduce_scatter", "all_gather")), "allreduce"),
                op=next((t for t in rest if t in ("max", "avg")), "sum"),
                rsteps=next((int(t[1:]) for t in rest if t.startswith("S")), 0),
                factors=next(([int(v) for v in t[1:].split("x")] for t in rest if t.startswith("Z")), None))


# ar_kernel_of's answer -> the kernel function it launches
KERNEL_NAMES = {
    "AR_KERNEL_NONE": None, "AR_KERNEL_DIRECT": "k_direct", "AR_KERNEL_LITERAL": "k_literal",
    "AR_KERNEL_REPLAY": "k_fused", "AR_KERNEL_STAGED": "k_fused_staged", "AR_KERNEL_STRIDED": "k_fused_strided",
    "AR_KERNEL_FIXED_CHAIN": "k_fused_fixed", "AR_KERNEL_FIXED_BALANCED": "k_fused_fixed",
    "AR_KERNEL_FIXED_STACK": "k_fused_fixed", "AR_KERNEL_MULTI": "k_fused_multi", "AR_KERNEL_ROWS": "k_fused_rows",
    "AR_KERNEL_ROWS_VEC": "k_fused_rows_vec", "AR_KERNEL_DAG": "k_fused_dag", "AR_KERNEL_JIT": "ar_jit",
}


def profile_name(wl_name, P):
    """A workload's name in profile summaries and traffic records: the name, and
    the rank count where it is not the workload's default (small_batch_P3)."""
    return wl_name if P is None or P == WORKLOADS[wl_name]["P"] else f"{wl_name}_P{P}"


def load_traffic(wl_name, key):
    """The committed counter summary's record for this workload and schedule:
    HBM bytes per launch (FETCH_SIZE and WRITE_SIZE, each scaled by what it
    reads for a plain copy of known size) and the kernel the trace names; None
    when the summary was taken from a different kernel source."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    try:
        with open(path) as f:
            t = json.load(f)
    except (OSError, ValueError):
        return None
    if t.get("kernel_hash") != kernel_source_hash():
        return None
    return t.get("entries", {}).get(f"{wl_name}/{key}")


def reporter(A, call, wl, measured=None):
    """The cost reporter's view of one call: method steps, the busiest rank's
    elements and bytes sent, all ranks' bytes, the bytes each executor moves
    through HBM, and the process cost model's predicted time of literal
    execution (one launch per step) beside the measured literal time."""
    s = A.ar_schedule_build(call)
    info = s.info()
    c = s.cost()
    elt = ELT[wl["dtype"]] * wl["batch"]
    _, _, t = A.ar_select(call)
    out = {"steps": info.steps, "sent_busiest_elems": c.sent_busiest, "recv_busiest_elems": c.recv_busiest,
           "reduced_busiest_elems": c.reduced_busiest, "max_rank_sent_bytes": c.max_rank_sent * elt,
           "sent_total_bytes": c.sent_total * elt, "literal_hbm_bytes": c.literal_hbm_bytes,
           "fused_hbm_bytes": c.fused_hbm_bytes, "model_literal_us": round(t * 1e6, 3)}
    if measured is not None:
        out["measured_literal_us"] = round(measured * 1e3, 3)
        out["model_over_measured"] = round(t * 1e6 / (measured * 1e3), 4) if measured > 0 else None
    return out


def run_schedules(r, entries, steps, warmup, steps_others, warm=False, log=None):
    """Time every schedule entry; returns {key: row}."""
    A = r.A
    out = {}
    for i, e in enumerate(entries):
        key = schedule_key(*e)
        q = parse_key(key)
        row = r.time(q["algo"], q["knob"], q["ex"], steps if i == 0 else steps_others, warmup if i == 0 else 2,
                     coll=q["coll"], op=q["op"], rsteps=q["rsteps"], factors=q["factors"])
        if warm:
            row["warm_GBps"] = r.time(q["algo"], q["knob"], q["ex"], steps_others, 2, cold=False, kernel_pass=False,
                                      coll=q["coll"], op=q["op"], rsteps=q["rsteps"], factors=q["factors"])["GBps"]
        call = r.call_for(q["algo"], q["knob"], q["ex"], coll=q["coll"], op=q["op"], rsteps=q["rsteps"],
                          factors=q["factors"])
        row["kernel"] = KERNEL_NAMES[A.ar_kernel_of(call).name]
        row["pct_hbm_peak"] = round(100.0 * row["GBps"] / HBM_PEAK_GBPS, 2)
        row["kernel_pct_hbm_peak"] = round(100.0 * row["kernel_GBps"] / HBM_PEAK_GBPS, 2)
        row["report"] = reporter(A, call, r.wl, row["ms"] if q["ex"] == "literal" else None)
        for k in list(row):
            if isinstance(row[k], float):
                row[k] = round(row[k], 5 if "ms" in k else 2)
        out[key] = row
        if log:
            print(f"bench: {r.wl['name']} P={r.wl['P']} {key}: {row['GBps']} GB/s ({row['kernel']})",
                  file=sys.stderr, flush=True)
    return out


def extra_workload(name, flush, P=None, unbatched=False):
    """One of the other workloads: its schedules, fewer steps, same method."""
    import torch
    wl = workload(name, P)
    x = make_inputs(wl)
    r = Runner(wl, x, flush)
    steps = wl.get("steps", 20)
    # the 8-rank workload fits the Infinity Cache: its warm figures beside the cold ones
    rows = run_schedules(r, wl["entries"], steps, 3, steps, warm=wl.get("warm", False), log=True)
    out = {"workload": workload_label(wl), "P": wl["P"], "n": wl["n"],
           "batch": wl["batch"], "steps": steps, "schedules": rows}
    if unbatched:
        algo, knob = wl["entries"][0][:2]
        out["unbatched"] = r.unbatched(algo, knob, wl["batch"])
    del r, x
    torch.cuda.empty_cache()
    return out


# --------------------------------------------------------------------------
# rocprofv3 output -> profiles/ summaries
# --------------------------------------------------------------------------
PROFILE_COMMANDS = """command (kernel trace):
  rocprofv3 --kernel-trace --stats -d {root}/{case}/trace -o t --output-format csv -- python3 bench.py --workload {wl}{popt} --schedule {key} --steps 30 --warmup 5 --no-cpu --no-extras > {root}/{case}/bench.json
commands (counters, one pass each):
  rocprofv3 --pmc FETCH_SIZE -d {root}/{case}/fetch -o c --output-format csv -- python3 bench.py --workload {wl}{popt} --schedule {key} --steps 3 --warmup 1 --no-cpu --no-extras
  rocprofv3 --pmc WRITE_SIZE -d {root}/{case}/write -o c --output-format csv -- python3 bench.py --workload {wl}{popt} --schedule {key} --steps 3 --warmup 1 --no-cpu --no-extras
  rocprofv3 --pmc {sq} -d {root}/{case}/sq -o c --output-format csv -- python3 bench.py --workload {wl}{popt} --schedule {key} --steps 3 --warmup 1 --no-cpu --no-extras
  rocprofv3 --pmc FETCH_SIZE -d {root}/calib/fetch -o c --output-format csv -- python3 bench.py --calibrate-copy 512
  rocprofv3 --pmc WRITE_SIZE -d {root}/calib/write -o c --output-format csv -- python3 bench.py --calibrate-copy 512
summary:
  python3 bench.py --summarize-profiles {root}"""


# the shader-sequencer counters of the profile's third pass (at most 8 SQ
# counters fit one pass)
SQ_COUNTERS = ("SQ_WAVES", "SQ_INSTS_VALU", "SQ_INSTS_SALU", "SQ_INSTS_LDS", "SQ_LDS_BANK_CONFLICT",
               "SQ_WAVE_CYCLES", "SQ_BUSY_CYCLES", "SQ_WAIT_INST_LDS")


def _csv_rows(pattern):
    rows = []
    for path in sorted(glob.glob(pattern, recursive=True)):
        with open(path, newline="") as f:
            rows += list(csv.DictReader(f))
    return rows


def _col(row, *names):
    low = {k.lower(): v for k, v in row.items()}
    for n in names:
        if n.lower() in low:
            return low[n.lower()]
    raise KeyError(f"none of {names} in {list(row)}")


def _counter_kib(dirpath, counter):
    """Per kernel name: mean counter value per dispatch (KiB), and dispatches."""
    acc = {}
    for row in _csv_rows(os.path.join(dirpath, "**", "*counter_collection.csv")):
        if _col(row, "Counter_Name") != counter:
            continue
        name = _col(row, "Kernel_Name")
        disp = _col(row, "Dispatch_Id", "Correlation_Id")
        acc.setdefault(name, {}).setdefault(disp, 0.0)
        acc[name][disp] += float(_col(row, "Counter_Value"))
    return {k: (statistics.fmean(v.values()), len(v)) for k, v in acc.items()}


def _counters(dirpath, kernel):
    """Mean value per dispatch of every counter recorded for `kernel`."""
    acc = {}
    for row in _csv_rows(os.path.join(dirpath, "**", "*counter_collection.csv")):
        if _col(row, "Kernel_Name") != kernel:
            continue
        name = _col(row, "Counter_Name")
        disp = _col(row, "Dispatch_Id", "Correlation_Id")
        acc.setdefault(name, {}).setdefault(disp, 0.0)
        acc[name][disp] += float(_col(row, "Counter_Value"))
    return {k: statistics.fmean(v.values()) for k, v in acc.items()}


def _kernel_stats(dirpath):
    rows = _csv_rows(os.path.join(dirpath, "**", "*kernel_stats.csv"))
    out = []
    for row in rows:
        out.append(dict(name=_col(row, "Name", "KernelName", "Kernel_Name"), calls=int(float(_col(row, "Calls"))),
                        avg_us=float(_col(row, "AverageNs", "Average_Ns")) / 1e3,
                        min_us=float(_col(row, "MinNs", "Min_Ns")) / 1e3,
                        max_us=float(_col(row, "MaxNs", "Max_Ns")) / 1e3))
    return sorted(out, key=lambda r: -r["calls"] * r["avg_us"])


def _short_kernel(name):
    """'void ar::k_fused_fixed<1, 0, 3, 2, 7>(ar::FixPtrs, ...)' -> 'k_fused_fixed'."""
    base = name.split("(")[0].split("<")[0]
    return base.split("::")[-1].split()[-1]


def summarize_profiles(root):
    """Write profiles/<kernel>_<workload>[_<schedule>].txt and profiles/traffic.json
    from rocprofv3 CSV output laid out as in PROFILE_COMMANDS: root/calib/{fetch,write}
    for the counter scale factors, and per case root/<case>/{trace,fetch,write} plus
    the bench line the traced run printed (bench.json)."""
    calib_bytes = 512 << 20
    fetch_cal = _counter_kib(os.path.join(root, "calib", "fetch"), "FETCH_SIZE")
    write_cal = _counter_kib(os.path.join(root, "calib", "write"), "WRITE_SIZE")
    cal_f = max(fetch_cal.values())[0] if fetch_cal else None
    cal_w = max(write_cal.values())[0] if write_cal else None
    fetch_scale = calib_bytes / 1024 / cal_f if cal_f else None
    write_scale = calib_bytes / 1024 / cal_w if cal_w else None
    traffic = {"kernel_hash": kernel_source_hash(), "fetch_scale": fetch_scale and round(fetch_scale, 5),
               "write_scale": write_scale and round(write_scale, 5),
               "calibration": f"plain device copy of 512 MiB (bench.py --calibrate-copy 512): FETCH_SIZE "
                              f"{cal_f and round(cal_f, 1)} KiB, WRITE_SIZE {cal_w and round(cal_w, 1)} KiB per "
                              f"dispatch", "entries": {}}
    os.makedirs(os.path.join(ROOT, "profiles"), exist_ok=True)
    written = []
    for case in sorted(os.listdir(root)):
        cdir = os.path.join(root, case)
        bj = os.path.join(cdir, "bench.json")
        if case == "calib" or not os.path.isdir(cdir) or not os.path.exists(bj):
            continue
        with open(bj) as f:
            line = json.loads([ln for ln in f if ln.startswith("{")][-1])
        wl0 = line["config"]["workload"].split(":")[0]
        P = line["config"].get("P")
        wl = profile_name(wl0, P)
        popt = "" if wl == wl0 else f" --P {P}"
        key = line["config"]["schedule"]
        alg = line["roofline"]["algorithmic_bytes_per_launch"]
        stats = _kernel_stats(os.path.join(cdir, "trace"))
        dom_name = line["roofline"]["kernel"]
        dom = next((s for s in stats if _short_kernel(s["name"]) == dom_name), None)
        if dom is None:
            print(f"summarize: no {dom_name} in the trace of {case}", file=sys.stderr)
            continue
        fetch = _counter_kib(os.path.join(cdir, "fetch"), "FETCH_SIZE").get(dom["name"])
        write = _counter_kib(os.path.join(cdir, "write"), "WRITE_SIZE").get(dom["name"])
        launches = line["roofline"].get("launches_per_call", 1)
        lines = [f"# {dom_name} on {line['config']['workload']}; schedule {key}",
                 f"# kernel source hash {traffic['kernel_hash']}", "",
                 PROFILE_COMMANDS.format(root=root.rstrip("/"), case=case, wl=wl0, popt=popt, key=key,
                                         sq=" ".join(SQ_COUNTERS)), "",
                 "kernel stats (rocprofv3 --stats, all kernels of the run):",
                 f"  {'name':70s} {'calls':>6s} {'avg_us':>9s} {'min_us':>9s} {'max_us':>9s}"]
        for s in stats[:6]:
            lines.append(f"  {s['name'][:70]:70s} {s['calls']:6d} {s['avg_us']:9.2f} {s['min_us']:9.2f} "
                         f"{s['max_us']:9.2f}")
        ach = alg / launches / (dom["avg_us"] * 1e-6) / 1e9
        lines += ["", f"dominant kernel: {dom['name'].split('(')[0].replace('void ', '')}",
                  f"  average duration {dom['avg_us']:.2f} us over {dom['calls']} dispatches",
                  f"  algorithmic bytes per launch: {alg / launches:.0f}",
                  f"  achieved = algorithmic / average duration = {ach:.1f} GB/s = {100 * ach / HBM_PEAK_GBPS:.1f}% "
                  f"of 8 TB/s",
                  f"  bench.py line under the profiler: value {line['value']} GB/s, ms_per_step {line['ms_per_step']},"
                  f" roofline.achieved {line['roofline']['achieved']} GB/s (library events)"]
        entry = {"kernel": dom["name"].split("(")[0].replace("void ", ""), "avg_kernel_ns": round(dom["avg_us"] * 1e3, 1),
                 "dispatches": dom["calls"], "algorithmic_bytes_per_launch": alg / launches}
        if fetch and write and fetch_scale and write_scale:
            tb = fetch[0] * 1024 * fetch_scale + write[0] * 1024 * write_scale
            entry.update(fetch_kib_per_dispatch=round(fetch[0], 2), write_kib_per_dispatch=round(write[0], 2),
                         bytes_per_launch=int(tb))
            lines += ["", "HBM traffic (per dispatch):",
                      f"  FETCH_SIZE {fetch[0]:.1f} KiB x {fetch_scale:.4f} + WRITE_SIZE {write[0]:.1f} KiB x "
                      f"{write_scale:.4f} = {tb:.0f} bytes",
                      f"  traffic / algorithmic = {tb / (alg / launches):.4f}",
                      f"  scale factors from a plain 512 MiB device copy: FETCH_SIZE reads {cal_f:.0f} KiB, "
                      f"WRITE_SIZE {cal_w:.0f} KiB for 524288 KiB moved each way"]
        sq = _counters(os.path.join(cdir, "sq"), dom["name"])
        if sq.get("SQ_WAVES"):
            waves = sq["SQ_WAVES"]
            lines += ["", "shader sequencer (per dispatch; per wave where it is a count of instructions):"]
            for c in SQ_COUNTERS:
                if c in sq:
                    per = f"  ({sq[c] / waves:.1f} per wave)" if c.startswith("SQ_INSTS") else ""
                    lines.append(f"  {c:22s} {sq[c]:14.0f}{per}")
            if "SQ_INSTS_LDS" in sq and "SQ_LDS_BANK_CONFLICT" in sq:
                lines.append(f"  LDS bank-conflict cycles per LDS instruction: "
                             f"{sq['SQ_LDS_BANK_CONFLICT'] / max(sq['SQ_INSTS_LDS'], 1):.2f}")
            entry["sq"] = {c: round(sq[c]) for c in SQ_COUNTERS if c in sq}
        traffic["entries"][f"{wl}/{key}"] = entry
        safe = key.replace("/", "_")
        path = os.path.join(ROOT, "profiles", f"{dom_name}_{wl}_{safe}.txt")
        with open(path, "w") as f:
            f.write("\n".join(lines) + "\n")
        written.append(path)
    with open(os.path.join(ROOT, "profiles", "traffic.json"), "w") as f:
        json.dump(traffic, f, indent=1)
    print(json.dumps({"written": [os.path.relpath(p, ROOT) for p in written], "traffic_entries": len(traffic["entries"])}))


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed calls of the headline schedule (default 20; 50 for the small-message batch)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="prime_fp32", choices=sorted(WORKLOADS))
    ap.add_argument("--P", type=int, default=None, help="ranks of the small_batch workload (3, 6, 12 or 24)")
    ap.add_argument("--headline-only", action="store_true", help="time only the headline schedule")
    ap.add_argument("--schedule", default=None, metavar="KEY",
                    help="time this schedule as the headline, a key of the schedule table such as "
                         "ring/r0/fused/reduce_scatter or generalized/r0/literal/S6 (for profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--no-extras", action="store_true", help="skip the other workloads")
    ap.add_argument("--warm", action="store_true", help="also report warm-cache (no flush) figures")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run one plain device copy of MIB MiB (for counter scaling) and exit")
    ap.add_argument("--latency", action="store_true",
                    help="per-call device time of single small Allreduces (graph replay) and exit")
    ap.add_argument("--model", action="store_true",
                    help="fit alpha/beta/gamma to literal-mode (one launch per step) timings and check "
                         "the model's choice of schedule and knob against measurement")
    ap.add_argument("--summarize-profiles", default=None, metavar="DIR",
                    help="write profiles/*.txt and profiles/traffic.json from rocprofv3 output under DIR and exit")
    args = ap.parse_args()

    if args.summarize_profiles:
        summarize_profiles(args.summarize_profiles)
        return

    if args.gpus != 1:
        print(f"bench.py measures one GPU: the library runs every rank of an Allreduce as a buffer "
              f"in one GPU's HBM and has no multi-GPU path (asked for --gpus {args.gpus})", file=sys.stderr)
        sys.exit(2)

    import torch
    assert torch.cuda.is_available(), "bench.py needs an MI355X"
    torch.cuda.set_device(0)

    if args.calibrate_copy:
        nbytes = args.calibrate_copy << 20
        a = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        torch.cuda.synchronize()
        b.copy_(a)
        torch.cuda.synchronize()
        print(json.dumps({"calibration_copy_bytes": nbytes}))
        return

    if args.latency:
        print(json.dumps(latency()))
        return

    if args.model:
        model_fit(args)
        return

    import allreduce_schedule_algorithms_amd as A
    wl = workload(args.workload, args.P)
    flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB, written before every step
    x = make_inputs(wl)
    r = Runner(wl, x, flush)
    entries = wl["entries"]
    if args.schedule:
        q = parse_key(args.schedule)
        entries = [(q["algo"], q["knob"], q["ex"], q["coll"], q["op"], q["rsteps"], q["factors"])]
    elif args.headline_only:
        entries = entries[:1]
    if args.steps is None:
        args.steps = wl.get("steps", 20)
    steps_others = max(10, args.steps) if "steps" in wl else 20
    schedules = run_schedules(r, entries, args.steps, args.warmup, steps_others,
                              warm=args.warm or (wl.get("warm", False) and not args.schedule),
                              log=not args.schedule)
    hkey = schedule_key(*entries[0])
    head = schedules[hkey]
    h = parse_key(hkey)
    ceiling = r.ceiling() if not args.schedule and not args.headline_only else None

    call = r.call_for(h["algo"], h["knob"], h["ex"], coll=h["coll"], op=h["op"], rsteps=h["rsteps"],
                      factors=h["factors"])
    cst = A.ar_schedule_build(call).cost()
    value = head["GBps"]
    achieved = head["kernel_GBps"]
    rec = load_traffic(profile_name(wl["name"], wl["P"]), hkey)
    traffic = rec.get("bytes_per_launch") if rec else None
    alg = essential_bytes(wl, h["coll"])
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": head["kernel"],
                "avg_launch_ms": head["kernel_ms"],
                "launches_per_call": 1 if h["ex"] != "literal" else A.ar_schedule_build(call).info().steps,
                "algorithmic_bytes_per_launch": alg,
                "model_bytes_per_launch": cst.fused_hbm_bytes if h["ex"] != "literal" else cst.literal_hbm_bytes}
    if ceiling:
        roofline["frac_of_best_2P_ceiling"] = round(achieved / ceiling["best_2P"], 4)

    cpu = None if args.no_cpu else cpu_baseline(wl, x)
    del x
    line = {
        "metric": "allreduce essential GB/s (P·n in + P·n out) and % of HBM peak, per schedule",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": head["ms"],
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": DT_NAME[wl["dtype"]],
        "data": "synthetic",
        "config": {"workload": workload_label(wl),
                   "P": wl["P"], "n": wl["n"], "batch": wl["batch"], "schedule": hkey, "knob": h["knob"],
                   "exec": h["ex"], "cache": "cold (1 GiB flush before each step)",
                   "value_statistic": "median of the timed calls"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "wall_ms_per_step": head["wall_ms_per_step"],
        "roofline": roofline,
        "ceiling": ceiling,
        "cpu_baseline": cpu,
        "schedules": schedules,
    }
    if not args.schedule and not args.headline_only and not args.no_extras:
        del r
        torch.cuda.empty_cache()
        extra = {}
        for name in EXTRA_WORKLOADS:
            if name == "small_batch":
                for P in SMALL_BATCH_P:
                    extra[f"small_batch_P{P}"] = extra_workload(name, flush, P, unbatched=(P == 24))
            else:
                extra[name] = extra_workload(name, flush)
        line["extra"] = extra
    print(json.dumps(line))


if __name__ == "__main__":
    main()
