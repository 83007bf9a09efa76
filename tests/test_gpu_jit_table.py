"""GPU parity of the table form of the compiled kernel (AR_KERNEL_JIT on programs
of one range and one result tree over more than 32 ranks): the tree's shape
compiled once as straight-line code, the leaf and output ranks read from a
table, one work item per wave. Bit-exact against the CPU oracle for halving and
doubling with fold-in, recursive doubling, the binomial tree, the pipelined
chain and the generalized algorithm over 2^8 ranks; every dtype and operation;
aligned buffers (vector items, with masked partial vectors at a ragged end),
unaligned buffers (element items), batches of short instances, and sampled
offsets of 192 x 2^20 bf16 in the launch the benchmark times."""
import numpy as np
import pytest

import oracle
from synth import inputs
from gpu_util import bits, gpu_allreduce

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def _kernel(P, n, dtype, op, algo, knob, batch=1):
    import allreduce_schedule_algorithms_amd as A
    return A.ar_kernel_of(A.make_call(P, n, dtype, op, algo, knob, batch=batch))


CASES = [  # P, algo, knob
    (33, "rh_rd", 0), (33, "chain", 8), (63, "binomial", 0), (100, "rd", 0), (100, "rh_rd", 0),
    (127, "chain", 1), (192, "rh_rd", 0), (192, "binomial", 0), (256, "generalized", 0),
]
TYPES = [("int32", "sum"), ("int32", "max"), ("fp32", "max"), ("fp32", "avg"), ("bf16", "sum"), ("bf16", "avg")]


@pytest.mark.parametrize("P,algo,knob", CASES)
def test_table_form_one_range_schedules(P, algo, knob):
    import allreduce_schedule_algorithms_amd as A
    for i, (dtype, op) in enumerate(TYPES):
        if (P + i) % 2:  # every case runs half of the dtype/op pairs (all of them over the cases)
            continue
        for n, mis in ((4099, False), (4099, True), (9000, False)):
            assert _kernel(P, n, dtype, op, algo, knob) == A.Kernel.AR_KERNEL_JIT, (P, algo, n, dtype)
            x = inputs.make(dtype, P, n, seed=P * 7 + n + i)
            want = oracle.allreduce(x, algo, dtype, op, knob=knob)
            got = gpu_allreduce(x, algo, dtype, op, knob, "fused", misalign=mis)
            assert np.array_equal(bits(got), bits(want)), (P, algo, knob, dtype, op, n, mis)


def test_table_form_batches_of_short_instances():
    import allreduce_schedule_algorithms_amd as A
    for P, n, B, algo, knob, dtype, op in ((63, 106, 200, "binomial", 0, "fp32", "sum"),
                                           (127, 300, 20, "chain", 1, "bf16", "max"),
                                           (40, 1000, 9, "rd", 0, "int32", "sum")):
        assert _kernel(P, n, dtype, op, algo, knob, B) == A.Kernel.AR_KERNEL_JIT, (P, n, B)
        x = inputs.make(dtype, P, n * B, seed=P + n + B)
        want = oracle.allreduce(x.reshape(P, B, n), algo, dtype, op, knob=knob, n=n)
        for mis in (False, True):
            got = gpu_allreduce(x, algo, dtype, op, knob, "fused", batch=B, misalign=mis)
            assert np.array_equal(bits(got.reshape(P, B, n)), bits(want)), (P, n, B, algo, dtype, op, mis)


def test_table_form_full_size_sampled():
    # the 192-rank bf16 halving + doubling at 2^20 elements as the benchmark
    # launches it (two vectors per lane), and a ragged 127-rank fp32 call;
    # sampled offsets (every part of the buffer) against the oracle
    import allreduce_schedule_algorithms_amd as A
    for P, n, algo, dtype, op in ((192, 1 << 20, "rh_rd", "bf16", "sum"), (127, (1 << 21) + 37, "rd", "fp32", "max")):
        assert _kernel(P, n, dtype, op, algo, 0) == A.Kernel.AR_KERNEL_JIT, (P, n, algo)
        x = inputs.make(dtype, P, n, seed=P + 3)
        idx = inputs.sample_indices(n, P, count=2048)
        want = oracle.allreduce(np.ascontiguousarray(x[:, idx]), algo, dtype, op, n=n, idx=idx)
        got = gpu_allreduce(x, algo, dtype, op, 0, "fused")
        assert np.array_equal(bits(got[:, idx]), bits(want)), (P, n, algo, dtype, op)
