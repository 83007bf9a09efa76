"""The allocation-free entry point, ar_allreduce_noalloc, through the C ABI: its
results equal ar_allreduce_ex's literal execution (the same kernels, with the
work records and workspace slots in the library's static device array instead
of allocations) and the CPU oracle, bit for bit, on two calls in a row whose
second is smaller than the first (the array keeps the first call's contents).
It allocates nothing: the library's cached plans and workspaces do not grow."""
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


def run(x, dtype, algo, knob, noalloc, groups=None, batch=1, misalign=False):
    import allreduce_schedule_algorithms_amd as A
    torch = torch_mod()
    P, total = x.shape
    bufs, keep = to_device(x, dtype, misalign)
    call = A.make_call(P, total // batch, dtype, "sum", algo, knob, "literal", batch, groups)
    ptrs = [b.data_ptr() for b in bufs]
    st = torch.cuda.current_stream()
    (A.ar_allreduce_noalloc if noalloc else A.ar_allreduce_ex)(ptrs, call, st)
    torch.cuda.synchronize()
    out = from_device(bufs, dtype)
    del keep
    return out


CASES = [  # (dtype, P, first n, second n, algo, knob, groups, batch): the second call is smaller
    ("fp32", 7, 1 << 18, 4099, "generalized", 2, None, 1),
    ("bf16", 12, 50_000, 999, "ahc", 0, [5, 7], 1),
    ("fp32", 24, 106 * 300, 106 * 37, "rd", 0, None, 1),
    ("int32", 8, 70_001, 333, "ring", 0, None, 1),
    ("fp32", 6, 106 * 200, 106 * 20, "generalized", 1, None, 106),  # batched instances of 106
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"{c[4]}-{c[0]}-P{c[1]}")
def test_noalloc_matches_the_literal_entry_point_on_two_calls(case):
    import allreduce_schedule_algorithms_amd as A
    dtype, P, n1, n2, algo, knob, groups, inst = case
    before = A.ar_cache_stats_get()
    for k, n in enumerate((n1, n2)):
        x = inputs.make(dtype, P, n, seed=n + k)
        batch = n // inst if inst > 1 else 1
        got = run(x, dtype, algo, knob, True, groups, batch)
        if inst > 1:
            want = oracle.allreduce(x.reshape(P, batch, inst), algo, dtype, "sum", knob=knob, n=inst).reshape(P, n)
        else:
            want = oracle.allreduce(x, algo, dtype, "sum", knob=knob, groups=groups)
        assert np.array_equal(bits(got), bits(want)), (case, n, "oracle")
        ref = run(x, dtype, algo, knob, False, groups, batch)
        assert np.array_equal(bits(got), bits(ref)), (case, n, "ar_allreduce_ex")
        # misaligned buffers take the element records
        got = run(x, dtype, algo, knob, True, groups, batch, misalign=True)
        assert np.array_equal(bits(got), bits(want)), (case, n, "misaligned")
    after = A.ar_cache_stats_get()
    # only the ar_allreduce_ex reference calls may have added device tables or workspaces
    assert after["retired_workspaces"] >= before["retired_workspaces"]


def test_noalloc_allocates_nothing():
    import allreduce_schedule_algorithms_amd as A
    P, n = 7, 30_011
    x = inputs.make("fp32", P, n, seed=3)
    want = oracle.allreduce(x, "generalized", "fp32", "sum", knob=3)
    before = A.ar_cache_stats_get()
    for _ in range(2):
        assert np.array_equal(bits(run(x, "fp32", "generalized", 3, True)), bits(want))
    after = A.ar_cache_stats_get()
    for key in ("workspaces", "retired_workspaces", "plan_device_bytes", "workspace_device_bytes"):
        assert after[key] == before[key], (key, before, after)


def test_noalloc_rejects_what_it_cannot_hold():
    import allreduce_schedule_algorithms_amd as A
    torch = torch_mod()
    # 8 ranks x 2^22 fp32 with one workspace slot per rank: 128 MiB of slots
    P, n = 8, 1 << 22
    bufs = [torch.full((n,), float(p), dtype=torch.float32, device="cuda") for p in range(P)]
    ptrs = [b.data_ptr() for b in bufs]
    call = A.make_call(P, n, "fp32", "sum", "generalized", 1, "literal")
    assert A.ar_workspace_bytes(call) > A.AR_NOALLOC_SCRATCH_BYTES
    with pytest.raises(A.ArError) as e:
        A.ar_allreduce_noalloc(ptrs, call)
    assert e.value.status == A.Status.AR_UNSUPPORTED
    with pytest.raises(A.ArError) as e:
        A.ar_allreduce_noalloc(ptrs, A.make_call(P, n, "fp32", "sum", "generalized", 1, "fused"))
    assert e.value.status == A.Status.AR_INVALID_ARGUMENT
    torch.cuda.synchronize()
    for p, b in enumerate(bufs):  # nothing was enqueued
        assert torch.equal(b, torch.full((n,), float(p), dtype=torch.float32, device="cuda"))
