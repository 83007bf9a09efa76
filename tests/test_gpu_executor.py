"""GPU checks of the executor's memory lifetime: captured HIP graphs stay valid
while the library builds many more plans and grows its workspaces, a first call
inside a capture is refused without touching anything, and literal calls that
bring no workspace run concurrently on two streams without sharing partials.
Every result is compared bit for bit with the CPU oracle."""
import numpy as np
import pytest

import oracle
from synth import inputs
from gpu_util import bits, from_device, to_device, torch_mod

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def test_captured_graph_survives_300_new_plans():
    import allreduce_schedule_algorithms_amd as A
    torch = torch_mod()
    P, n, B = 7, 1000, 4
    # the literal calls need workspace slots (several result vectors per step)
    cases = [("generalized", 2, "fused"), ("generalized", 1, "literal"), ("generalized", 3, "literal")]
    x = inputs.make("fp32", P, n * B, seed=11)
    want = [oracle.allreduce(x.reshape(P, B, n), algo, "fp32", "sum", knob=knob, n=n).reshape(P, B * n)
            for algo, knob, _ in cases]
    st = torch.cuda.Stream()
    dev = [to_device(x, "fp32")[0] for _ in cases]
    pristine = [[b.clone() for b in d] for d in dev]
    calls = [A.make_call(P, n, "fp32", "sum", algo, knob, ex) for algo, knob, ex in cases]
    ptrs = [[[b.data_ptr() + i * n * 4 for b in d] for i in range(B)] for d in dev]

    def restore():
        with torch.cuda.stream(st):
            for d, p0 in zip(dev, pristine):
                for b, q in zip(d, p0):
                    b.copy_(q)
        torch.cuda.synchronize()

    def run_all():
        for c, pp in zip(calls, ptrs):
            for i in range(B):
                A.ar_allreduce_ex(pp[i], c, st)

    with torch.cuda.stream(st):  # eager calls build the plans and the stream's literal workspace
        run_all()
    torch.cuda.synchronize()
    for c, d, w in zip(cases, dev, want):
        assert np.array_equal(bits(from_device(d, "fp32")), bits(w)), (c, "eager")
    restore()
    stats0 = A.ar_cache_stats_get()
    g = torch.cuda.CUDAGraph()
    refused = None
    with torch.cuda.graph(g, stream=st):
        run_all()
        # a schedule and size not seen before needs device tables: refused, nothing enqueued
        try:
            A.ar_allreduce_ex(ptrs[0][0], A.make_call(P, n - 1, "fp32", "sum", "ring", 0, "fused"), st)
        except A.ArError as e:
            refused = e
    assert refused is not None and refused.status == A.Status.AR_UNSUPPORTED, refused
    # 300 new plans on the same stream, and a literal call large enough to make
    # the stream's workspace grow (the captured calls' workspace is retired, not freed)
    scratch = [torch.zeros(8192, dtype=torch.float32, device="cuda") for _ in range(P)]
    sp = [b.data_ptr() for b in scratch]
    with torch.cuda.stream(st):
        for k in range(300):
            A.ar_allreduce_ex(sp, A.make_call(P, 2000 + k, "fp32", "sum", "generalized", 1, "fused"), st)
        A.ar_allreduce_ex(sp, A.make_call(P, 8192, "fp32", "sum", "generalized", 1, "literal"), st)
    torch.cuda.synchronize()
    stats1 = A.ar_cache_stats_get()
    assert stats1["retired_plans"] > stats0["retired_plans"]
    assert stats1["retired_workspaces"] > stats0["retired_workspaces"]
    for rep in range(3):
        restore()
        g.replay()
        torch.cuda.synchronize()
        for c, d, w in zip(cases, dev, want):
            assert np.array_equal(bits(from_device(d, "fp32")), bits(w)), (c, rep)
    del g


def test_literal_calls_on_two_streams_keep_their_partials_apart():
    # calls without a workspace on two streams at once: each stream has its own
    # workspace, so interleaved launches never mix partial results
    import allreduce_schedule_algorithms_amd as A
    torch = torch_mod()
    P, n = 12, 1 << 16
    runs = [("generalized", 2), ("generalized", 3)]  # both need workspace slots
    xs = [inputs.make("fp32", P, n, seed=21 + i) for i in range(len(runs))]
    wants = [oracle.allreduce(x, algo, "fp32", "sum", knob=k) for x, (algo, k) in zip(xs, runs)]
    streams = [torch.cuda.Stream() for _ in runs]
    devs = [to_device(x, "fp32") for x in xs]
    pristine = [[b.clone() for b in d[0]] for d in devs]
    calls = [A.make_call(P, n, "fp32", "sum", algo, k, "literal") for algo, k in runs]
    for rep in range(5):
        for d, p0, s in zip(devs, pristine, streams):
            with torch.cuda.stream(s):
                for b, q in zip(d[0], p0):
                    b.copy_(q)
        torch.cuda.synchronize()
        for _ in range(3):  # the launches of both streams interleave on the device
            for d, c, s in zip(devs, calls, streams):
                A.ar_allreduce_ex([b.data_ptr() for b in d[0]], c, s)
            torch.cuda.synchronize()
            for d, p0, s in zip(devs, pristine, streams):
                with torch.cuda.stream(s):
                    for b, q in zip(d[0], p0):
                        b.copy_(q)
            torch.cuda.synchronize()
        for d, c, s in zip(devs, calls, streams):
            A.ar_allreduce_ex([b.data_ptr() for b in d[0]], c, s)
        torch.cuda.synchronize()
        for d, want, run in zip(devs, wants, runs):
            assert np.array_equal(bits(from_device(d[0], "fp32")), bits(want)), (run, rep)
