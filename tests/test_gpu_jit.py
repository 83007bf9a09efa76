"""GPU parity of the compiled register DAG (AR_KERNEL_JIT): several result trees
per range (or a latency-bound call) over at most 32 ranks, each range's DAG written out as straight-line
register code and compiled for the schedule at run time. Bit-exact against the
CPU oracle, every dtype and operation, aligned and unaligned buffers (vector
and element paths), one and two vectors per thread, batches of long ranges."""
import numpy as np
import pytest

import oracle
from oracle import numerics as nu
from synth import inputs
from gpu_util import bits, gpu_allreduce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def _kernel(P, n, dtype, algo, r, batch=1, steps=0):
    import allreduce_schedule_algorithms_amd as A
    return A.ar_kernel_of(A.make_call(P, n, dtype, "sum", algo, r, batch=batch, steps=steps))


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
def test_jit_every_multi_tree_schedule(dtype):
    import allreduce_schedule_algorithms_amd as A
    ops = ("sum", "max") + (("avg",) if dtype != "int32" else ())
    ran = 0
    for algo in ("generalized", "generalized_xor"):
        for P in (3, 5, 7, 8, 12, 16):
            if algo == "generalized_xor" and P & (P - 1):
                continue
            for r in range(1, nu.ceil_log2(P) + 1):
                for n, mis in ((37, False), (4099, False), (4099, True), (70001, False)):
                    if _kernel(P, n, dtype, algo, r) != A.Kernel.AR_KERNEL_JIT:
                        continue
                    x = inputs.make(dtype, P, n, seed=P * 11 + n + r)
                    for op in ops:
                        want = oracle.allreduce(x, algo, dtype, op, knob=r)
                        got = gpu_allreduce(x, algo, dtype, op, r, "fused", misalign=mis)
                        assert np.array_equal(bits(got), bits(want)), (algo, dtype, P, n, mis, r, op)
                    ran += 1
    assert ran >= 20, ran  # the compiled form is what these schedules run


def test_jit_batches_and_more_steps():
    # batches of instances whose ranges are long enough for per-instance items,
    # a schedule with more than 8 result trees per range (13 ranks, r = 4 of 4
    # steps), and bf16 max where one vector per thread fits the register budget
    cases = [(7, 700, "generalized", 2, 9, 0, "fp32", "sum"), (5, 640, "generalized", 1, 13, 0, "int32", "max"),
             (13, 1000, "generalized", 4, 1, 4, "fp32", "sum"), (7, 1 << 16, "generalized", 2, 1, 0, "bf16", "max"),
             (12, 3001, "generalized", 2, 2, 0, "bf16", "avg")]
    import allreduce_schedule_algorithms_amd as A
    for i, (P, n, algo, r, B, steps, dtype, op) in enumerate(cases):
        assert _kernel(P, n, dtype, algo, r, B, steps) == A.Kernel.AR_KERNEL_JIT, (P, n, r, B)
        x = inputs.make(dtype, P, n * B, seed=500 + i)
        want = oracle.allreduce(x.reshape(P, B, n), algo, dtype, op, knob=r, n=n, steps=steps or None)
        for mis in (False, True):
            got = gpu_allreduce(x, algo, dtype, op, r, "fused", batch=B, misalign=mis, steps=steps)
            assert np.array_equal(bits(got.reshape(P, B, n)), bits(want)), (P, n, r, B, dtype, op, mis)


def test_jit_two_vectors_per_thread_sampled():
    # calls of at least 2^20 vectors take two vectors per thread where the live
    # values fit; sampled offsets against the oracle (every part of the buffer)
    import allreduce_schedule_algorithms_amd as A
    for P, r, dtype, op in ((7, 2, "int32", "max"), (5, 1, "fp32", "avg"), (6, 2, "fp32", "sum")):
        n = (1 << 22) + 40
        assert _kernel(P, n, dtype, "generalized", r) == A.Kernel.AR_KERNEL_JIT
        x = inputs.make(dtype, P, n, seed=P + r)
        idx = inputs.sample_indices(n, P, count=4096)
        want = oracle.allreduce(np.ascontiguousarray(x[:, idx]), "generalized", dtype, op, knob=r, n=n, idx=idx)
        got = gpu_allreduce(x, "generalized", dtype, op, r, "fused")
        assert np.array_equal(bits(got[:, idx]), bits(want)), (P, r, dtype, op)

