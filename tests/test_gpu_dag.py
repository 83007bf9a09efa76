"""GPU parity of the DAG replay (AR_KERNEL_DAG): every distinct combination of a
range's result trees evaluated once, values in LDS. AR_EXEC_DAG forces it for
every schedule; fused execution picks it for ranges with more result trees than
the register replays hold (the generalized algorithm with large r at P = 63,
100, 127). Bit-exact against the CPU oracle."""
import numpy as np
import pytest

import oracle
from oracle import numerics as nu
from synth import inputs
from gpu_util import bits, gpu_allreduce, torch_mod

pytestmark = pytest.mark.gpu

ALGOS = ("direct", "ring", "rh_rd", "rd", "binomial", "generalized", "generalized_xor", "ahc", "chain")


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def knobs(algo, P):
    if algo.startswith("generalized"):
        return range(nu.ceil_log2(P) + 1)
    return [3] if algo == "chain" else [0]


def groups_for(algo, P):
    return [P // 3 + 1, P - (P // 3 + 1)] if algo == "ahc" else None


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_dag_every_schedule(algo, dtype):
    ops = ("sum", "max") + (("avg",) if dtype != "int32" else ())
    for P in (3, 5, 8, 12):
        if algo == "generalized_xor" and P & (P - 1):
            continue
        for n, mis in ((37, False), (4099, False), (4099, True), (70001, False)):
            ks = list(knobs(algo, P))
            for r in (ks if n < 70001 else sorted({ks[0], ks[-1]})):
                x = inputs.make(dtype, P, n, seed=P * 7 + n + r)
                for op in ops:
                    want = oracle.allreduce(x, algo, dtype, op, knob=r, groups=groups_for(algo, P))
                    got = gpu_allreduce(x, algo, dtype, op, r, "dag", groups_for(algo, P), misalign=mis)
                    assert np.array_equal(bits(got), bits(want)), (algo, dtype, P, n, mis, r, op)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_dag_127_ranks_every_r(dtype):
    # the generalized paper's experiment size: the fused call runs one launch at every r
    import allreduce_schedule_algorithms_amd as A
    P = 127
    for n in (106, 4099):
        x = inputs.make(dtype, P, n, seed=n)
        for r in range(8):
            want = oracle.allreduce(x, "generalized", dtype, "sum", knob=r)
            k = A.ar_kernel_of(A.make_call(P, n, dtype, "sum", "generalized", r))
            assert k != A.Kernel.AR_KERNEL_LITERAL, (n, r, k)
            if r >= 4:
                assert k == A.Kernel.AR_KERNEL_DAG, (n, r, k)
            got = gpu_allreduce(x, "generalized", dtype, "sum", r, "fused")
            assert np.array_equal(bits(got), bits(want)), (dtype, n, r)


def test_dag_127_ranks_large_sampled():
    # 127 ranks x 2^16: every element within the normwise tolerance of fp64 and
    # every rank's sampled offsets equal to the oracle's replay of the schedule
    P, n = 127, 1 << 16
    x = inputs.make("fp32", P, n, seed=5)
    idx = inputs.sample_indices(n, P, count=2048)
    ref = nu.fp64_reference(x, "fp32")
    for r in (4, 5, 6, 7):
        got = gpu_allreduce(x, "generalized", "fp32", "sum", r, "fused")
        want = oracle.allreduce(x[:, idx], "generalized", "fp32", "sum", knob=r, n=n, idx=idx)
        assert np.array_equal(bits(got[:, idx]), bits(want)), r
        for p in range(P):
            assert nu.normwise_rel_error(got[p], ref) <= 1e-5, (r, p)


def test_dag_other_large_rank_counts():
    import allreduce_schedule_algorithms_amd as A
    for P in (63, 100):
        L = nu.ceil_log2(P)
        x = inputs.make("fp32", P, 106, seed=P)
        for r in range(L + 1):
            assert A.ar_kernel_of(A.make_call(P, 106, "fp32", "sum", "generalized", r)) != A.Kernel.AR_KERNEL_LITERAL
            want = oracle.allreduce(x, "generalized", "fp32", "sum", knob=r)
            assert np.array_equal(bits(gpu_allreduce(x, "generalized", "fp32", "sum", r, "fused")), bits(want)), (P, r)


def test_dag_batches_steps_groups_and_halves():
    from oracle import schedules as sch
    P, n, B = 24, 106, 37
    x = inputs.make("fp32", P, n * B, seed=3, dist="uniform_pm1")
    for r in (0, 1, 3, 5):
        want = oracle.allreduce(x.reshape(P, B, n), "generalized", "fp32", "sum", knob=r, n=n).reshape(P, B * n)
        got = gpu_allreduce(x, "generalized", "fp32", "sum", r, "dag", batch=B)
        assert np.array_equal(bits(got), bits(want)), r
    for algo in ("ring", "rd", "binomial"):
        want = oracle.allreduce(x.reshape(P, B, n), algo, "fp32", "sum", n=n).reshape(P, B * n)
        assert np.array_equal(bits(gpu_allreduce(x, algo, "fp32", "sum", 0, "dag", batch=B)), bits(want)), algo
    P = 12
    x = inputs.make("fp32", P, 4099, seed=4)
    for r in (1, 3, 5):
        want = oracle.allreduce(x, "generalized", "fp32", "sum", knob=r, steps=5)
        assert np.array_equal(bits(gpu_allreduce(x, "generalized", "fp32", "sum", r, "dag", steps=5)), bits(want))
    for f in ((2, 6), (3, 4)):
        want = oracle.allreduce(x, "generalized", "fp32", "sum", knob=2, factors=f)
        assert np.array_equal(bits(gpu_allreduce(x, "generalized", "fp32", "sum", 2, "dag", list(f))), bits(want))
    own = np.arange(4099) // (-(-4099 // P))
    for algo in ("ring", "generalized", "direct"):
        want = sch.reduce_scatter(x, algo, "fp32", "sum")
        got = gpu_allreduce(x, algo, "fp32", "sum", 0, "dag", collective="reduce_scatter")
        assert np.array_equal(bits(got[own, np.arange(4099)]), bits(want)), algo
        want = sch.all_gather(x, algo, "fp32")
        assert np.array_equal(bits(gpu_allreduce(x, algo, "fp32", "sum", 0, "dag", collective="all_gather")),
                              bits(want)), algo


def test_dag_prime_fp32_full_size_sampled():
    # the 7-rank 2^24 workload with r = 3 (seven result trees per part) through
    # the DAG replay: sampled offsets against the oracle, every element against
    # the fp64 tolerance
    x = inputs.workload("prime_fp32")
    n = x.shape[1]
    idx = inputs.sample_indices(n, 7)
    got = gpu_allreduce(x, "generalized", "fp32", "sum", 3, "dag")
    want = oracle.allreduce(x[:, idx], "generalized", "fp32", "sum", knob=3, n=n, idx=idx)
    assert np.array_equal(bits(got[:, idx]), bits(want))
    ref = nu.fp64_reference(x, "fp32")
    for p in range(7):
        assert nu.normwise_rel_error(got[p], ref) <= 1e-5, p
