#!/usr/bin/env python3
"""Allreduce throughput on one MI355X: essential GB/s and % of HBM peak.

A step is one in-place Allreduce of P rank buffers resident in HBM (one call of
ar_allreduce_ex), timed with HIP events on the stream it is launched on. Before
every step, outside the timed region, the inputs are restored from a pristine
copy (in-place sums grow the values) and the 256 MB Infinity Cache is flushed
by writing a 1 GiB buffer, so each step starts cold from HBM.

Essential bytes = P * n * elt read + P * n * elt written (every input read
once, every output written once). value = essential bytes / mean time of the
call between two events (launch latency included); roofline.achieved =
essential bytes / mean device time of the call's kernel, from events the
library records around its own launch.

Default workload: 8 ranks x 2^20 fp32 N(0,1), recursive halving + doubling,
fused replay (the schedule the workload names), with ring, direct and
recursive doubling (fused and literal) reported beside it.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, vendor figure

WORKLOADS = {
    "rh_fp32": dict(
        desc="8 ranks x 2^20 fp32 N(0,1), seed 0",
        P=8, n=1 << 20, dtype="fp32", batch=1, groups=None,
        headline=("rh_rd", 0, "fused"),
        others=[("ring", 0, "fused"), ("direct", 0, "fused"), ("rd", 0, "fused"), ("generalized_xor", 0, "fused"),
                ("rh_rd", 0, "literal"), ("ring", 0, "literal"),
                ("rh_rd", 0, "fused", "reduce_scatter"), ("rh_rd", 0, "fused", "all_gather"),
                ("generalized", 0, "fused", "allreduce", "sum", 0, [2, 4]),
                ("generalized", 0, "fused", "allreduce", "sum", 0, [4, 2]),
                ("generalized", 0, "literal", "allreduce", "sum", 0, [4, 2])]),
    "prime_fp32": dict(
        desc="7 ranks x 2^24 fp32 N(0,1e-3), seed 0",
        P=7, n=1 << 24, dtype="fp32", batch=1, groups=None,
        headline=("generalized", 0, "fused"),
        others=[("generalized", 1, "fused"), ("generalized", 2, "fused"), ("generalized", 3, "fused"),
                ("ring", 0, "fused"), ("direct", 0, "fused"), ("ring", 0, "literal"), ("generalized", 0, "literal"),
                ("generalized", 0, "fused", "allreduce", "avg"),
                ("generalized", 0, "fused", "reduce_scatter"), ("ring", 0, "fused", "reduce_scatter"),
                ("direct", 0, "fused", "reduce_scatter"), ("generalized", 0, "literal", "reduce_scatter"),
                ("generalized", 0, "fused", "all_gather"), ("ring", 0, "fused", "all_gather"),
                ("direct", 0, "fused", "all_gather"), ("generalized", 0, "literal", "all_gather"),
                ("generalized", 0, "fused", "allreduce", "sum", 4), ("generalized", 0, "fused", "allreduce", "sum", 6),
                ("generalized", 0, "literal", "allreduce", "sum", 4),
                ("generalized", 0, "literal", "allreduce", "sum", 5),
                ("generalized", 0, "literal", "allreduce", "sum", 6),
                ("chain", 1, "fused"), ("chain", 8, "literal"), ("chain", 64, "literal")]),
    "ahc_bf16": dict(
        desc="192 ranks in groups (64, 128) x 2^20 bf16 N(0,1), fp32 accumulation, seed 0",
        P=192, n=1 << 20, dtype="bf16", batch=1, groups=[64, 128],
        headline=("ahc", 0, "fused"),
        others=[("direct", 0, "fused"), ("ahc", 0, "literal"), ("ahc", 0, "fused", "allreduce", "avg")]),
    "small_batch": dict(
        desc="24 ranks x 10^4 instances x 106 fp32 U(-1,1), seed 0",
        P=24, n=106, dtype="fp32", batch=10_000, groups=None, steps=100,
        headline=("rd", 0, "fused"),
        others=[("binomial", 0, "fused"), ("direct", 0, "fused"), ("generalized", 5, "fused"),
                ("generalized", 0, "fused"), ("ring", 0, "fused"),
                ("rd", 0, "literal"), ("binomial", 0, "literal"), ("generalized", 5, "literal"),
                ("generalized", 0, "literal")]),
    "ring_int32": dict(
        desc="5 ranks x 4096 int32 U[-2^20, 2^20], seed 0",
        P=5, n=4096, dtype="int32", batch=1, groups=None, steps=100,
        headline=("ring", 0, "fused"),
        others=[("direct", 0, "fused"), ("ring", 0, "literal")]),
}

DT_NAME = {"fp32": "f32", "bf16": "bf16", "int32": "i32"}
ELT = {"fp32": 4, "bf16": 2, "int32": 4}


def kernel_source_hash() -> str:
    """Hash of the device code and of the executor that lays out its work items."""
    h = hashlib.sha256()
    for name in ("kernels.h", "launch.h", "exec.hip"):
        with open(os.path.join(ROOT, "allreduce_schedule_algorithms_amd", "csrc", name), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


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
    def __init__(self, wl, x):
        import torch

        import allreduce_schedule_algorithms_amd as A
        self.A = A
        self.wl = wl
        self.stream = torch.cuda.Stream()
        self.pristine = host_to_device(x, wl["dtype"])           # (P, batch*n)
        self.work = torch.empty_like(self.pristine)
        self.flush = torch.empty(1 << 28, dtype=torch.float32, device="cuda")  # 1 GiB
        self.ptrs = [self.work[p].data_ptr() for p in range(wl["P"])]
        self.essential = essential_bytes(wl)
        self.kernel_events = KernelEvents()

    def call_for(self, algo, knob, ex, start_event=None, stop_event=None, coll="allreduce", op="sum", rsteps=0,
                 factors=None):
        wl = self.wl
        return self.A.make_call(wl["P"], wl["n"], wl["dtype"], op, algo, knob, ex, wl["batch"],
                                wl["groups"] if algo == "ahc" else factors,
                                start_event=start_event, stop_event=stop_event, collective=coll, steps=rsteps)

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

        def prep():
            with torch.cuda.stream(st):
                self.work.copy_(self.pristine)
                if cold:
                    self.flush.zero_()

        for _ in range(warmup):
            prep()
            self.A.ar_allreduce_ex(self.ptrs, plain, st)
        call_evs = [(ev(), ev()) for _ in range(steps)]
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for k in range(steps):
            prep()
            call_evs[k][0].record(st)
            self.A.ar_allreduce_ex(self.ptrs, plain, st)
            call_evs[k][1].record(st)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        ms = [a.elapsed_time(b) for a, b in call_evs]
        mean = statistics.fmean(ms)
        out = dict(ms=mean, ms_median=statistics.median(ms), ms_min=min(ms), wall_ms_per_step=1e3 * wall / steps,
                   GBps=essential / (mean * 1e-3) / 1e9)
        if kernel_pass:
            kev = self.kernel_events
            kern_evs = [(kev.create(), kev.create()) for _ in range(steps)]
            calls = [self.call_for(algo, knob, ex, a, b, coll, op, rsteps, factors) for a, b in kern_evs]
            torch.cuda.synchronize()
            for k in range(steps):
                prep()
                self.A.ar_allreduce_ex(self.ptrs, calls[k], st)
            torch.cuda.synchronize()
            kmean = statistics.fmean([kev.elapsed_ms(a, b) for a, b in kern_evs])
            kev.destroy(kern_evs)
            out.update(kernel_ms=kmean, kernel_GBps=essential / (kmean * 1e-3) / 1e9)
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
        ptr_sets = [[p + b * wl["n"] * elt for p in self.ptrs] for b in range(calls)]
        with torch.cuda.stream(st):
            self.work.copy_(self.pristine)
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
               "wall_us_per_call": round(wall * 1e6 / calls, 3), "schedule": f"{algo}/r{knob}/fused"}
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
        return out

    def copy_ceiling(self, gib=2):
        import torch
        a = torch.empty(gib << 28, dtype=torch.float32, device="cuda")
        b = torch.empty_like(a)
        a.fill_(1.0)
        for _ in range(2):
            b.copy_(a)
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        s.record()
        reps = 5
        for _ in range(reps):
            b.copy_(a)
        e.record()
        torch.cuda.synchronize()
        t = s.elapsed_time(e) / reps * 1e-3
        del a, b
        return 2.0 * (gib << 30) / t / 1e9


def cpu_baseline(wl, x, budget_s=12.0):
    """The oracle, as it stands, on this host: repeated replays of the headline schedule."""
    import numpy as np

    import oracle
    algo, knob, _ = wl["headline"]
    P, n, B = wl["P"], wl["n"], wl["batch"]
    if B > 1:
        xs = x.reshape(P, B, n)
        sample = f"full workload ({B} instances of {n})"
        ess = 2.0 * P * n * B * ELT[wl["dtype"]]
        idx = None
    elif P * n > (1 << 24):
        # bounded sample: every rank's first 2^20 offsets' worth, spread over the buffer
        from synth import inputs
        idx = np.unique(np.linspace(0, n - 1, num=min(n, (1 << 24) // P), dtype=np.int64))
        xs = np.ascontiguousarray(x[:, idx])
        sample = f"{len(idx)} of {n} offsets per rank (evenly spaced, all parts covered)"
        ess = 2.0 * P * len(idx) * ELT[wl["dtype"]]
        del inputs
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
            "sample": f"{sample}; {algo} replay, {len(times)} runs, mean {mean:.3f} s (NumPy, one thread); "
                      f"host {host_cpu()}",
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
]


def latency(calls=2000):
    """Per-call device time of single small Allreduces: `calls` calls on
    consecutive instances, captured once in a HIP graph and replayed, timed
    with events around the replay. Without the host's enqueue cost this is the
    library's alpha on this device (launch, one kernel, completion)."""
    import numpy as np
    import torch

    import allreduce_schedule_algorithms_amd as A
    from synth import inputs
    rows = []
    for P, n, algo, knob in LATENCY_CASES:
        x = inputs.make("fp32", P, n * calls, seed=1)
        bufs = [torch.from_numpy(np.ascontiguousarray(x[p])).cuda() for p in range(P)]
        call = A.make_call(P, n, "fp32", "sum", algo, knob)
        st = torch.cuda.Stream()
        ptrs = [[b.data_ptr() + i * n * 4 for b in bufs] for i in range(calls)]
        with torch.cuda.stream(st):
            for i in range(20):  # plans built outside the capture
                A.ar_allreduce_ex(ptrs[i], call, st)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for i in range(calls):
                A.ar_allreduce_ex(ptrs[i], call, st)
        g.replay()
        torch.cuda.synchronize()
        a, z = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        with torch.cuda.stream(st):
            a.record(st)
            g.replay()
            z.record(st)
        torch.cuda.synchronize()
        rows.append({"P": P, "n": n, "schedule": f"{algo}/r{knob}/fused", "kernel": KERNEL_NAMES[A.ar_kernel_of(call).name],
                     "us_per_call": round(a.elapsed_time(z) * 1e3 / calls, 3)})
        del g, bufs
    print(json.dumps({"latency_fp32_graph_replay": rows, "calls": calls}))


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
    "AR_KERNEL_FIXED_STACK": "k_fused_fixed", "AR_KERNEL_MULTI": "k_fused_multi", "AR_KERNEL_ROWS": "k_fused_rows", "AR_KERNEL_ROWS_VEC": "k_fused_rows_vec",
}


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


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed calls per schedule (default 50; 100 for the latency-bound workloads)")
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="rh_fp32", choices=sorted(WORKLOADS))
    ap.add_argument("--headline-only", action="store_true", help="time only the headline schedule")
    ap.add_argument("--schedule", default=None, metavar="KEY",
                    help="time this schedule as the headline, a key of the schedule table such as "
                         "ring/r0/fused/reduce_scatter or generalized/r0/literal/S6 (for profiling)")
    ap.add_argument("--no-cpu", action="store_true", help="skip the oracle timing")
    ap.add_argument("--warm", action="store_true", help="also report warm-cache (no flush) figures")
    ap.add_argument("--calibrate-copy", type=int, default=0, metavar="MIB",
                    help="run one plain device copy of MIB MiB (for counter scaling) and exit")
    ap.add_argument("--latency", action="store_true",
                    help="per-call device time of single small Allreduces (graph replay) and exit")
    ap.add_argument("--model", action="store_true",
                    help="fit alpha/beta/gamma to literal-mode (one launch per step) timings and check "
                         "the model's choice of schedule and knob against measurement")
    args = ap.parse_args()

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
        latency()
        return

    if args.model:
        model_fit(args)
        return

    wl = dict(WORKLOADS[args.workload])
    wl["name"] = args.workload
    x = make_inputs(wl)
    r = Runner(wl, x)
    hkey = args.schedule or schedule_key(*wl["headline"])
    h = parse_key(hkey)
    algo, knob, ex = h["algo"], h["knob"], h["ex"]

    def timed(key, steps, warmup, **kw):
        q = parse_key(key)
        return r.time(q["algo"], q["knob"], q["ex"], steps, warmup, coll=q["coll"], op=q["op"], rsteps=q["rsteps"],
                      factors=q["factors"], **kw)

    if args.steps is None:
        args.steps = wl.get("steps", 50)
    # the other schedules: half the headline's calls, at least 20 (all of them
    # where the workload asks for many calls per schedule)
    other_steps = args.steps if "steps" in wl else max(20, args.steps // 2)
    head = timed(hkey, args.steps, args.warmup)
    schedules = {hkey: head}
    if not args.headline_only and not args.schedule:
        for entry in wl["others"]:
            key = schedule_key(*entry)
            schedules[key] = timed(key, other_steps, 2)
    if args.warm:
        for key in list(schedules):
            schedules[key]["warm_GBps"] = timed(key, other_steps, 2, cold=False, kernel_pass=False)["GBps"]
    for v in schedules.values():
        v["pct_hbm_peak"] = round(100.0 * v["GBps"] / HBM_PEAK_GBPS, 2)
        for k in ("ms", "ms_median", "ms_min", "kernel_ms", "wall_ms_per_step", "GBps", "kernel_GBps"):
            if k in v:
                v[k] = round(v[k], 5 if "ms" in k else 2)
    ceiling = r.copy_ceiling()
    unbatched = None
    if wl["batch"] > 1 and not args.schedule and not args.headline_only:
        unbatched = r.unbatched(algo, knob, wl["batch"])

    # model bytes from the library's cost walk (fused / literal HBM bytes per call)
    import allreduce_schedule_algorithms_amd as A
    s = A.ar_schedule_build(r.call_for(algo, knob, ex, coll=h["coll"], op=h["op"], rsteps=h["rsteps"],
                                       factors=h["factors"]))
    cst = s.cost()
    value = head["GBps"]
    achieved = head["kernel_GBps"]
    rec = load_traffic(args.workload, hkey)
    traffic = rec.get("bytes_per_launch") if rec else None
    # the kernel the library picks for this call (its own answer, host side)
    kind = A.ar_kernel_of(r.call_for(algo, knob, ex, coll=h["coll"], op=h["op"], rsteps=h["rsteps"],
                                     factors=h["factors"]))
    kernel = KERNEL_NAMES[kind.name]
    roofline = {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": traffic,
                "kernel": kernel,
                "avg_launch_ms": head["kernel_ms"],
                "algorithmic_bytes_per_launch": essential_bytes(wl, h["coll"]),
                "model_bytes_per_launch": cst.fused_hbm_bytes if ex != "literal" else cst.literal_hbm_bytes}

    cpu = None if args.no_cpu else cpu_baseline(wl, x)
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
        "config": {"workload": f"{args.workload}: {wl['desc']}", "P": wl["P"], "n": wl["n"], "batch": wl["batch"],
                   "schedule": hkey, "knob": knob, "exec": ex, "cache": "cold (1 GiB flush before each step)"},
        "pct_hbm_peak": round(100.0 * value / HBM_PEAK_GBPS, 2),
        "runtime_copy_GBps": round(ceiling, 1),  # torch D2D copy of 2 GiB (HIP runtime blit), context only
        "wall_ms_per_step": head["wall_ms_per_step"],
        "roofline": roofline,
        "cpu_baseline": cpu,
        "schedules": schedules,
    }
    if unbatched:
        line["unbatched"] = unbatched
    print(json.dumps(line))


if __name__ == "__main__":
    main()
