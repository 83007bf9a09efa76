"""GPU parity: the HIP path, called through the C ABI, against the CPU oracle.

Bit-exact for every schedule, dtype and op (int32 and max reach the plain
result; fp32 / bf16 sums must reproduce the oracle's replay of the same
schedule), plus the normwise tolerance against an fp64 reference
(1e-5 fp32, 8e-3 bf16) at the full workload sizes, where the oracle is
evaluated on sampled offsets (every part boundary included).
"""
import numpy as np
import pytest

import oracle
from oracle import numerics as nu
from synth import inputs
from gpu_util import bits, from_device, gpu_allreduce, to_device, torch_mod

pytestmark = pytest.mark.gpu

ALGOS = ("direct", "ring", "rh_rd", "rd", "binomial", "generalized", "generalized_xor", "ahc")
FP_TOL = {"fp32": 1e-5, "bf16": 8e-3}


@pytest.fixture(scope="module", autouse=True)
def _need_gpu():
    import torch
    assert torch.cuda.is_available(), "GPU tests need a visible MI355X"
    torch.cuda.set_device(0)


def knobs(algo, P):
    return range(nu.ceil_log2(P) + 1) if algo.startswith("generalized") else [0]


def groups_for(algo, P):
    if algo != "ahc":
        return None
    return [P] if P < 3 else [P // 3 + 1, P - (P // 3 + 1)]


def check_tol(y, x, dtype):
    ref = nu.fp64_reference(x, dtype)
    for p in range(y.shape[0]):
        yp = nu.bf16_to_f32(y[p]) if dtype == "bf16" else y[p]
        assert nu.normwise_rel_error(yp, ref) <= FP_TOL[dtype], p


# --------------------------------------------------------------------------
# every schedule x dtype x op x execution mode, small ragged sizes
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS)
def test_small_all_schedules(algo, dtype):
    for P in (3, 5, 7, 8, 12):
        if algo == "generalized_xor" and P & (P - 1):
            continue
        for n in (37, 4099):
            for r in knobs(algo, P):
                x = inputs.make(dtype, P, n, seed=P * 7 + n)
                for op in ("sum", "max"):
                    want = oracle.allreduce(x, algo, dtype, op, knob=r, groups=groups_for(algo, P))
                    for ex in ("fused", "literal", "replay"):
                        got = gpu_allreduce(x, algo, dtype, op, r, ex, groups_for(algo, P))
                        assert np.array_equal(bits(got), bits(want)), (ex, algo, dtype, P, n, r, op)


@pytest.mark.parametrize("algo", ["direct", "ring", "rd", "generalized", "ahc"])
def test_misaligned_buffers_take_element_path(algo):
    P, n = 6, 1000
    for dtype in ("fp32", "bf16"):
        x = inputs.make(dtype, P, n, seed=3)
        for r in knobs(algo, P):
            want = oracle.allreduce(x, algo, dtype, "sum", knob=r, groups=groups_for(algo, P))
            for ex in ("fused", "literal"):
                got = gpu_allreduce(x, algo, dtype, "sum", r, ex, groups_for(algo, P), misalign=True)
                assert np.array_equal(bits(got), bits(want)), (algo, dtype, r, ex)


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
def test_perfect_binary_trees(dtype):
    # schedules whose every tree is a perfect binary tree of 4 or 8 leaves run
    # the level-by-level kernel (vector and element paths, 2 or 4 vectors per
    # thread by size); the halves and batches as well
    import allreduce_schedule_algorithms_amd as A
    from oracle import schedules as sch
    ops = ("sum", "max") + (("avg",) if dtype != "int32" else ())
    for P in (4, 8):
        for algo, groups in (("rh_rd", None), ("rd", None), ("generalized_xor", None), ("generalized", [2, P // 2])):
            info = A.ar_schedule_build(A.make_call(P, 4099, dtype, "sum", algo, groups=groups)).info()
            assert info.max_trees == 1 and info.max_leaves == P
            for n, mis in ((37, False), (4099, True), (1 << 17, False), (3 << 20, False)):
                x = inputs.make(dtype, P, n, seed=P + n)
                for op in ops:
                    want = oracle.allreduce(x, algo, dtype, op, factors=groups if algo == "generalized" else None)
                    got = gpu_allreduce(x, algo, dtype, op, 0, "fused", groups, misalign=mis)
                    assert np.array_equal(bits(got), bits(want)), (P, algo, n, mis, op)
        x = inputs.make(dtype, P, 4099 * 3, seed=P)
        want = sch.reduce_scatter(x.reshape(P, 3, 4099), "rh_rd", dtype, "sum")
        got = gpu_allreduce(x, "rh_rd", dtype, "sum", 0, "fused", batch=3, collective="reduce_scatter")
        own = half_owner(4099, P)
        assert np.array_equal(bits(got.reshape(P, 3, 4099)[own, :, np.arange(4099)].T), bits(want)), P


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
def test_chain_trees(dtype):
    # schedules whose every tree is a chain of 2..8 leaves (ring, pipelined
    # chain) run the fixed-shape kernel; the reduce-scatter half as well
    from oracle import schedules as sch
    ops = ("sum", "max") + (("avg",) if dtype != "int32" else ())
    for P in (2, 3, 5, 7, 8):
        for algo, knob in (("ring", 0), ("chain", 1), ("chain", 3)):
            for n, mis in ((37, False), (4099, True), (1 << 17, False), (3 << 20, False)):
                x = inputs.make(dtype, P, n, seed=P * 3 + n)
                for op in ops:
                    want = oracle.allreduce(x, algo, dtype, op, knob=knob)
                    got = gpu_allreduce(x, algo, dtype, op, knob, "fused", misalign=mis)
                    assert np.array_equal(bits(got), bits(want)), (P, algo, knob, n, mis, op)
        x = inputs.make(dtype, P, 4099 * 3, seed=P)
        want = sch.reduce_scatter(x.reshape(P, 3, 4099), "ring", dtype, "sum")
        got = gpu_allreduce(x, "ring", dtype, "sum", 0, "fused", batch=3, collective="reduce_scatter")
        own = half_owner(4099, P)
        assert np.array_equal(bits(got.reshape(P, 3, 4099)[own, :, np.arange(4099)].T), bits(want)), P
        for n, mis in ((4099, True), (1 << 17, False)):  # the all-gather's single-leaf copies
            x = inputs.make(dtype, P, n, seed=P + 2 * n)
            want = sch.all_gather(x, "ring", dtype)
            got = gpu_allreduce(x, "ring", dtype, "sum", 0, "fused", misalign=mis, collective="all_gather")
            assert np.array_equal(bits(got), bits(want)), (P, n, mis)


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
def test_one_shape_per_program(dtype):
    # single-tree programs of at most 8 ranges whose trees all share one shape
    # that is neither a chain nor a perfect binary tree (the generalized
    # algorithm over Z_P, recursive doubling and halving with fold-in, the
    # binomial tree, AHC with small groups): the register-stack replay, beside
    # the fixed-shape kernel's Z_4 x Z_2 case
    from oracle import schedules as sch
    ops = ("sum", "max") + (("avg",) if dtype != "int32" else ())
    cases = [(7, "generalized", None), (5, "generalized", None), (6, "generalized", None), (6, "rd", None),
             (7, "binomial", None), (5, "rh_rd", None), (6, "ahc", [2, 4]), (8, "generalized", [4, 2])]
    for P, algo, groups in cases:
        for n, mis in ((37, False), (4099, True), (1 << 17, False), (3 << 20, False)):
            x = inputs.make(dtype, P, n, seed=P * 5 + n)
            for op in ops:
                want = oracle.allreduce(x, algo, dtype, op, groups=groups if algo == "ahc" else None,
                                        factors=groups if algo == "generalized" else None)
                got = gpu_allreduce(x, algo, dtype, op, 0, "fused", groups, misalign=mis)
                assert np.array_equal(bits(got), bits(want)), (P, algo, groups, n, mis, op)
    x = inputs.make(dtype, 7, 4099 * 3, seed=7)
    want = sch.reduce_scatter(x.reshape(7, 3, 4099), "generalized", dtype, "sum")
    got = gpu_allreduce(x, "generalized", dtype, "sum", 0, "fused", batch=3, collective="reduce_scatter")
    own = half_owner(4099, 7)
    assert np.array_equal(bits(got.reshape(7, 3, 4099)[own, :, np.arange(4099)].T), bits(want))


@pytest.mark.parametrize("algo", ["ring", "rh_rd", "binomial", "generalized", "ahc"])
def test_batched_instances(algo):
    P, n, B = 6, 53, 7
    x = inputs.make("fp32", P, B * n, seed=11, dist="uniform_pm1")
    for r in knobs(algo, P):
        want = oracle.allreduce(x.reshape(P, B, n), algo, "fp32", "sum", knob=r, groups=groups_for(algo, P),
                                n=n).reshape(P, B * n)
        for ex in ("fused", "literal"):
            got = gpu_allreduce(x, algo, "fp32", "sum", r, ex, groups_for(algo, P), batch=B)
            assert np.array_equal(bits(got), bits(want)), (algo, r, ex)


def test_most_ranks_and_tiny_buffers():
    for P in (2, 256):
        for n in (1, 3, 64):
            x = inputs.make("fp32", P, n, seed=P + n)
            for algo in ("direct", "ring", "rd", "binomial"):
                want = oracle.allreduce(x, algo, "fp32", "sum")
                for ex in ("fused", "literal"):
                    got = gpu_allreduce(x, algo, "fp32", "sum", 0, ex)
                    assert np.array_equal(bits(got), bits(want)), (P, n, algo, ex)


def test_many_tiny_chunks_pack_into_shared_workgroups():
    # P = 127 with a few hundred elements: thousands of 2-3 element chunks per
    # literal step, packed several to a workgroup; mixed with vector runs at
    # larger n
    P = 127
    for n in (256, 3000, 40_000):
        x = inputs.make("fp32", P, n, seed=n)
        cases = (("generalized", 0), ("ring", 0)) if n > 10_000 else \
            (("generalized", 0), ("generalized", 3), ("generalized", 7), ("ring", 0))
        for algo, r in cases:
            want = oracle.allreduce(x, algo, "fp32", "sum", knob=r)
            got = gpu_allreduce(x, algo, "fp32", "sum", r, "literal")
            assert np.array_equal(bits(got), bits(want)), (n, algo, r)


def test_max_signed_zeros_subnormals_infinities():
    # max is the total order with -0 < +0 on non-NaN values: ties between zeros
    # of both signs, subnormals next to zeros, infinities and repeated values,
    # in every kernel family that combines (fixed shapes, program-driven replay,
    # DAG, rows, direct, literal), fp32 and bf16
    pool = {"fp32": np.array([0.0, -0.0, 2.0**-149, -(2.0**-149), 2.0**-130, -(2.0**-130), 1.0, -1.0, np.inf,
                              -np.inf, 3.5, -3.5, 2.0**-149 * 7], dtype=np.float32),
            "bf16": np.array([0x0000, 0x8000, 0x0001, 0x8001, 0x0080, 0x8080, 0x3F80, 0xBF80, 0x7F80, 0xFF80,
                              0x4060, 0xC060, 0x0007], dtype=np.uint16)}
    rng = np.random.default_rng(11)
    cases = [(8, 4096, "rh_rd", 0, "fused", 1), (12, 3000, "ring", 0, "fused", 1), (24, 106, "generalized", 5, "fused", 40),
             (24, 106, "ring", 0, "fused", 60), (7, 5000, "generalized", 2, "fused", 1), (7, 999, "direct", 0, "fused", 1),
             (9, 777, "generalized", 3, "literal", 1), (63, 300, "generalized", 6, "fused", 1)]
    for P, n, algo, knob, ex, B in cases:
        for dtype in ("fp32", "bf16"):
            x = pool[dtype][rng.integers(0, len(pool[dtype]), size=(P, n * B))]
            want = oracle.allreduce(x.reshape(P, B, n) if B > 1 else x, algo, dtype, "max", knob=knob, n=n)
            got = gpu_allreduce(x, algo, dtype, "max", knob, ex, batch=B)
            assert np.array_equal(bits(got.reshape(np.shape(want))), bits(want)), (P, n, algo, knob, ex, dtype)


def test_side_stream_and_signed_zero():
    import torch
    s = torch.cuda.Stream()
    x = np.zeros((5, 300), dtype=np.float32)
    x[1] = -0.0
    x[4, ::2] = -0.0
    got = gpu_allreduce(x, "ring", "fp32", "max", stream=s)
    assert not np.signbit(got).any()
    x = inputs.make("fp32", 5, 300, seed=2)
    want = oracle.allreduce(x, "rh_rd", "fp32", "sum")
    assert np.array_equal(gpu_allreduce(x, "rh_rd", "fp32", "sum", stream=s), want)


# --------------------------------------------------------------------------
# the workloads at full size
# --------------------------------------------------------------------------
def test_ring_int32_5_ranks():
    x = inputs.workload("ring_int32")
    bf = nu.brute_force(x, "int32", "sum")
    for algo in ("ring", "direct"):
        for ex in ("fused", "literal"):
            got = gpu_allreduce(x, algo, "int32", "sum", 0, ex)
            assert np.array_equal(got, np.broadcast_to(bf, got.shape)), (algo, ex)


def test_rh_fp32_8_ranks():
    x = inputs.workload("rh_fp32")
    for algo in ("rh_rd", "ring", "direct", "rd"):
        want = oracle.allreduce(x, algo, "fp32", "sum")
        for ex in ("fused", "literal"):
            got = gpu_allreduce(x, algo, "fp32", "sum", 0, ex)
            assert np.array_equal(bits(got), bits(want)), (algo, ex)
            check_tol(got, x, "fp32")


def test_prime_fp32_7_ranks_sampled():
    x = inputs.workload("prime_fp32")
    P, n = x.shape
    idx = inputs.sample_indices(n, P, count=4096)
    xs = np.ascontiguousarray(x[:, idx])
    cases = [("generalized", r, "fused") for r in range(4)] + [("generalized", 0, "literal"),
                                                               ("generalized", 3, "literal"),
                                                               ("ring", 0, "fused"), ("direct", 0, "fused")]
    for algo, r, ex in cases:
        got = gpu_allreduce(x, algo, "fp32", "sum", r, ex)
        want = oracle.allreduce(xs, algo, "fp32", "sum", knob=r, n=n, idx=idx)
        assert np.array_equal(bits(got[:, idx]), bits(want)), (algo, r, ex)
        check_tol(got, x, "fp32")
        if r == 0 or algo != "generalized":
            assert (got == got[:1]).all()  # one tree per part: every rank holds the same bits


@pytest.mark.parametrize("P", [3, 6, 12, 24])
def test_small_batch_latency_path(P):
    x = inputs.workload("small_batch", P=P)
    B, ln = 10_000, 106
    for algo in ("rd", "binomial"):
        want = oracle.allreduce(x.reshape(P, B, ln), algo, "fp32", "sum", n=ln).reshape(P, B * ln)
        for ex in ("fused", "literal"):
            got = gpu_allreduce(x, algo, "fp32", "sum", 0, ex, batch=B)
            assert np.array_equal(bits(got), bits(want)), (algo, ex)
        check_tol(got, x, "fp32")


def test_ahc_bf16_192_ranks_sampled():
    x = inputs.workload("ahc_bf16")
    P, n = x.shape
    groups = [64, 128]
    idx = inputs.sample_indices(n, 256, count=2048)
    xs = np.ascontiguousarray(x[:, idx])
    for op in ("sum", "max"):
        want = oracle.allreduce(xs, "ahc", "bf16", op, groups=groups, n=n, idx=idx)
        for ex in ("fused", "literal"):
            got = gpu_allreduce(x, "ahc", "bf16", op, 0, ex, groups)
            assert np.array_equal(bits(got[:, idx]), bits(want)), (op, ex)
            assert (got == got[:1]).all()
            if op == "sum":
                check_tol(got, x, "bf16")
            else:
                assert np.array_equal(bits(got[0]), bits(nu.brute_force(x, "bf16", "max")))
    got = gpu_allreduce(x, "direct", "bf16", "sum")
    want = oracle.allreduce(xs, "direct", "bf16", "sum", n=n, idx=idx)
    assert np.array_equal(bits(got[:, idx]), bits(want))


def test_ring_halving_generalized_on_192_bf16_ranks_sampled():
    # the ring, recursive halving + doubling (128 ranks after folding in the 64
    # excess ones) and the generalized algorithm over Z_192 (r = 0, and r = 2)
    # on the 192-rank 2^20 bf16 workload: sampled offsets (every part boundary)
    # against the oracle, every element against the fp64 tolerance
    x = inputs.workload("ahc_bf16")
    P, n = x.shape
    idx = inputs.sample_indices(n, P, count=2048)
    xs = np.ascontiguousarray(x[:, idx])
    for algo, r, ex in (("ring", 0, "fused"), ("rh_rd", 0, "fused"), ("generalized", 0, "fused"),
                        ("generalized", 2, "fused"), ("ring", 0, "literal"), ("rh_rd", 0, "literal")):
        got = gpu_allreduce(x, algo, "bf16", "sum", r, ex)
        want = oracle.allreduce(xs, algo, "bf16", "sum", knob=r, n=n, idx=idx)
        assert np.array_equal(bits(got[:, idx]), bits(want)), (algo, r, ex)
        check_tol(got, x, "bf16")
        if r == 0:
            assert (got == got[:1]).all(), (algo, ex)  # one tree per part


# --------------------------------------------------------------------------
# model-driven choice: the call runs the schedule the oracle's model picks
# --------------------------------------------------------------------------
@pytest.mark.parametrize("form", ["all_ranks", "busiest"])
def test_auto_choice_runs_the_oracle_choice(form):
    import allreduce_schedule_algorithms_amd as A
    from oracle import cost
    try:
        if form == "busiest":
            A.ar_set_cost_model(2e-6, 1e-11, 2e-12, "busiest")
        m = A.ar_get_cost_model()
        for P in (5, 7, 8):
            for n in (64, 4099, 1 << 17):
                x = inputs.make("fp32", P, n, seed=P + n)
                for algo, knob in (("auto", 0), ("generalized", -1)):
                    a, r, _ = cost.select(P, n, "fp32", m["alpha"], m["beta"], m["gamma"], m["form"],
                                          algo=algo)
                    want = oracle.allreduce(x, a, "fp32", "sum", knob=r)
                    for ex in ("fused", "literal"):
                        got = gpu_allreduce(x, algo, "fp32", "sum", knob, ex)
                        assert np.array_equal(bits(got), bits(want)), (P, n, algo, a, r, ex)
    finally:
        A.ar_set_cost_model()


# --------------------------------------------------------------------------
# reduce-scatter / all-gather halves and avg
# --------------------------------------------------------------------------
HALVES = ("direct", "ring", "rh_rd", "generalized", "generalized_xor")


def half_owner(n, P):
    c = -(-n // P) if n else 1
    return np.arange(n) // c


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
@pytest.mark.parametrize("algo", HALVES)
def test_small_halves(algo, dtype):
    from oracle import schedules as sch
    for P in (2, 3, 5, 8, 12):
        if algo in ("rh_rd", "generalized_xor") and P & (P - 1):
            continue
        for n in (37, 4099):
            x = inputs.make(dtype, P, n, seed=P * 11 + n)
            own = half_owner(n, P)
            for op in ("sum", "max") + (("avg",) if dtype != "int32" else ()):
                want = sch.reduce_scatter(x, algo, dtype, op)
                for ex in ("fused", "literal", "replay"):
                    got = gpu_allreduce(x, algo, dtype, op, 0, ex, collective="reduce_scatter")
                    assert np.array_equal(bits(got[own, np.arange(n)]), bits(want)), (P, n, op, ex)
                    if ex == "fused":  # the rest of every buffer is untouched
                        keep = np.ones(x.shape, bool)
                        keep[own, np.arange(n)] = False
                        assert np.array_equal(bits(got)[keep], bits(x)[keep])
            want = sch.all_gather(x, algo, dtype)
            for ex in ("fused", "literal"):
                got = gpu_allreduce(x, algo, dtype, "sum", 0, ex, collective="all_gather")
                assert np.array_equal(bits(got), bits(want)), (P, n, ex)


@pytest.mark.parametrize("algo", ["direct", "ring", "rh_rd", "rd", "binomial", "generalized", "ahc"])
def test_small_allreduce_avg(algo):
    for P in (3, 5, 8):
        g = [P // 3 + 1, P - (P // 3 + 1)] if algo == "ahc" else None
        for dtype in ("fp32", "bf16"):
            for n in (37, 4099):
                x = inputs.make(dtype, P, n, seed=P + n)
                for r in knobs(algo, P):
                    want = oracle.allreduce(x, algo, dtype, "avg", knob=r, groups=g)
                    for ex in ("fused", "literal", "replay"):
                        got = gpu_allreduce(x, algo, dtype, "avg", r, ex, g)
                        assert np.array_equal(bits(got), bits(want)), (P, n, dtype, r, ex)


def test_halves_full_size_prime_ranks():
    # the 7-rank 2^24 fp32 workload through both halves, sampled oracle
    from oracle import schedules as sch
    x = inputs.workload("prime_fp32")
    P, n = x.shape
    idx = inputs.sample_indices(n, P, count=4096)
    xs = np.ascontiguousarray(x[:, idx])
    own = half_owner(n, P)[idx]
    for algo in ("ring", "generalized", "direct"):
        want = sch.reduce_scatter(xs, algo, "fp32", "sum", n=n, idx=idx)
        for ex in ("fused", "literal"):
            got = gpu_allreduce(x, algo, "fp32", "sum", 0, ex, collective="reduce_scatter")
            assert np.array_equal(bits(got[own, idx]), bits(want)), (algo, ex)
        got = gpu_allreduce(x, algo, "fp32", "sum", 0, "fused", collective="all_gather")
        assert np.array_equal(bits(got[:, idx]), bits(np.broadcast_to(x[own, idx], (P, len(idx))))), algo


# --------------------------------------------------------------------------
# the generalized algorithm with more than 2 ceil(log2 P) steps
# --------------------------------------------------------------------------
def test_generalized_more_steps_small():
    import allreduce_schedule_algorithms_amd as A
    for P in (5, 7, 12):
        L = nu.ceil_log2(P)
        for S in range(L, P):
            for r in sorted({0, 1, S}):
                for dtype in ("fp32", "bf16"):
                    for n in (37, 4099):
                        x = inputs.make(dtype, P, n, seed=S * 13 + r + n)
                        want = oracle.allreduce(x, "generalized", dtype, "sum", knob=r, steps=S)
                        for ex in ("fused", "literal"):
                            got = gpu_allreduce(x, "generalized", dtype, "sum", r, ex, steps=S)
                            assert np.array_equal(bits(got), bits(want)), (P, S, r, dtype, n, ex)


def test_fused_falls_back_to_literal_steps():
    # 255 ranks, r = 8: the DAG of a range holds more values than a workgroup's
    # LDS, so a fused call runs the literal steps (same bits) and takes the
    # caller's workspace when one is given
    import allreduce_schedule_algorithms_amd as A
    torch = torch_mod()
    P, n = 255, 600
    x = inputs.make("fp32", P, n, seed=41)
    want = oracle.allreduce(x, "generalized", "fp32", "sum", knob=8)
    call = A.make_call(P, n, "fp32", "sum", "generalized", 8)
    assert A.ar_kernel_of(call) == A.Kernel.AR_KERNEL_LITERAL
    assert np.array_equal(bits(gpu_allreduce(x, "generalized", "fp32", "sum", 8, "fused")), bits(want))
    need = A.ar_workspace_bytes(call)
    assert need > 0
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    bufs, keep = to_device(x, "fp32")
    short = A.make_call(P, n, "fp32", "sum", "generalized", 8, workspace=ws.data_ptr(), workspace_bytes=need - 1)
    with pytest.raises(A.ArError) as e:
        A.ar_allreduce_ex([b.data_ptr() for b in bufs], short, torch.cuda.current_stream())
    assert e.value.status == A.Status.AR_WORKSPACE_TOO_SMALL
    exact = A.make_call(P, n, "fp32", "sum", "generalized", 8, workspace=ws.data_ptr(), workspace_bytes=need)
    A.ar_allreduce_ex([b.data_ptr() for b in bufs], exact, torch.cuda.current_stream())
    torch.cuda.synchronize()
    assert np.array_equal(bits(from_device(bufs, "fp32")), bits(want))
    del keep


def test_generalized_more_steps_full_size_prime_ranks():
    x = inputs.workload("prime_fp32")
    P, n = x.shape
    idx = inputs.sample_indices(n, P, count=4096)
    xs = np.ascontiguousarray(x[:, idx])
    for S in (4, 5, 6):
        want = oracle.allreduce(xs, "generalized", "fp32", "sum", n=n, idx=idx, steps=S)
        for ex in ("fused", "literal"):
            got = gpu_allreduce(x, "generalized", "fp32", "sum", 0, ex, steps=S)
            assert np.array_equal(bits(got[:, idx]), bits(want)), (S, ex)
        check_tol(got, x, "fp32")


# --------------------------------------------------------------------------
# the generalized algorithm over other groups Z_m1 x ... x Z_mt
# --------------------------------------------------------------------------
def test_generalized_product_groups():
    import allreduce_schedule_algorithms_amd as A
    for P, fl in ((6, [(2, 3), (3, 2)]), (8, [(2, 4), (4, 2)]), (12, [(2, 6), (3, 4), (2, 2, 3)])):
        for f in fl:
            for r in (0, 1):
                for dtype in ("fp32", "bf16"):
                    for n in (37, 4099):
                        x = inputs.make(dtype, P, n, seed=P + r + n)
                        want = oracle.allreduce(x, "generalized", dtype, "sum", knob=r, factors=f)
                        for ex in ("fused", "literal"):
                            got = gpu_allreduce(x, "generalized", dtype, "sum", r, ex, groups=list(f))
                            assert np.array_equal(bits(got), bits(want)), (P, f, r, dtype, n, ex)


# --------------------------------------------------------------------------
# pipelined chain reduce + broadcast
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
def test_chain_small(dtype):
    for P in (2, 3, 5, 8, 12):
        for m in (1, 3, 16):
            for n in (37, 4099):
                x = inputs.make(dtype, P, n, seed=P * m + n)
                for op in ("sum", "max") + (("avg",) if dtype != "int32" else ()):
                    want = oracle.allreduce(x, "chain", dtype, op, knob=m)
                    for ex in ("fused", "literal"):
                        got = gpu_allreduce(x, "chain", dtype, op, m, ex)
                        assert np.array_equal(bits(got), bits(want)), (P, m, n, op, ex)


def test_chain_full_size_prime_ranks():
    x = inputs.workload("prime_fp32")
    P, n = x.shape
    idx = inputs.sample_indices(n, 64, count=4096)
    xs = np.ascontiguousarray(x[:, idx])
    for m in (1, 8, 64):
        want = oracle.allreduce(xs, "chain", "fp32", "sum", knob=m, n=n, idx=idx)
        for ex in ("fused", "literal"):
            got = gpu_allreduce(x, "chain", "fp32", "sum", m, ex)
            assert np.array_equal(bits(got[:, idx]), bits(want)), (m, ex)
        check_tol(got, x, "fp32")


def test_batched_halves_avg_and_chain():
    from oracle import schedules as sch
    P, n, B = 6, 106, 64
    x = inputs.make("fp32", P, n * B, seed=11)
    xb = x.reshape(P, B, n)
    own = half_owner(n, P)
    for ex in ("fused", "literal"):
        got = gpu_allreduce(x, "ring", "fp32", "sum", 0, ex, batch=B, collective="reduce_scatter").reshape(P, B, n)
        want = sch.reduce_scatter(xb, "ring", "fp32", "sum")
        assert np.array_equal(bits(got[own, :, np.arange(n)].T), bits(want)), ex
        got = gpu_allreduce(x, "generalized", "fp32", "sum", 0, ex, batch=B, collective="all_gather")
        assert np.array_equal(bits(got.reshape(P, B, n)), bits(sch.all_gather(xb, "generalized", "fp32"))), ex
        for algo, knob, op in (("rd", 0, "avg"), ("chain", 4, "sum"), ("generalized", 1, "avg")):
            got = gpu_allreduce(x, algo, "fp32", op, knob, ex, batch=B).reshape(P, B, n)
            want = oracle.allreduce(xb, algo, "fp32", op, knob=knob, n=n)
            assert np.array_equal(bits(got), bits(want)), (algo, op, ex)


def test_batched_short_ranges():
    # batches of short instances with chunked schedules: the fused replay runs
    # one strided item per range and block of instances; instance counts that
    # are not a multiple of the block, tiny n and misaligned buffers included
    cases = [(3, 106, "ring", 0, None), (7, 106, "generalized", 3, None), (24, 106, "generalized", 5, None),
             (24, 106, "generalized", 0, None), (6, 5, "rh_rd", 0, None), (5, 1, "ring", 0, None),
             (12, 106, "ahc", 0, [5, 7]), (8, 33, "chain", 3, None), (7, 106, "generalized", 1, None)]
    for i, (P, n, algo, knob, groups) in enumerate(cases):
        for dtype, op in (("fp32", "sum"), ("bf16", "sum"), ("int32", "max"), ("fp32", "avg")):
            B = 37 + i
            x = inputs.make(dtype, P, n * B, seed=100 + i)
            want = oracle.allreduce(x.reshape(P, B, n), algo, dtype, op, knob=knob, groups=groups, n=n)
            for ex, mis in (("fused", False), ("fused", True), ("literal", False)):
                got = gpu_allreduce(x, algo, dtype, op, knob, ex, groups, batch=B, misalign=mis)
                assert np.array_equal(bits(got.reshape(P, B, n)), bits(want)), (P, n, algo, knob, dtype, op, ex, mis)


def test_rows_kernel_batches():
    # batches of short instances whose ranges all run one program up to a
    # renaming of leaf ranks take k_fused_rows (one element per thread over the
    # whole batch, range and buffers looked up in LDS); several trees per range
    # take the DAG replay, other shapes keep the strided items. A tiny launch
    # limit splits one call into many launches, or leaves the vector form's
    # waves many positions each.
    import allreduce_schedule_algorithms_amd as A
    K = A.Kernel
    # fp32 calls of more than 4096 elements on aligned buffers run the vector
    # form (k_fused_rows_vec) for their whole vectors and k_fused_rows for a
    # ragged tail; bf16, misaligned buffers and tiny calls run k_fused_rows alone
    cases = [(24, 106, "generalized", 0, 10_000, K.AR_KERNEL_ROWS_VEC, (("fp32", "sum"),)),
             (24, 106, "ring", 0, 777, K.AR_KERNEL_ROWS_VEC, (("bf16", "sum"), ("int32", "max"), ("fp32", "avg"))),
             (12, 50, "generalized", 0, 301, K.AR_KERNEL_ROWS_VEC, (("fp32", "sum"), ("bf16", "avg"))),
             (6, 106, "ring", 0, 45, K.AR_KERNEL_ROWS_VEC, (("fp32", "sum"), ("int32", "sum"))),
             (24, 106, "ring", 0, 30, K.AR_KERNEL_ROWS, (("fp32", "sum"),)),
             (32, 70, "ring", 0, 99, K.AR_KERNEL_ROWS_VEC, (("fp32", "max"),)),
             (31, 200, "ring", 0, 41, K.AR_KERNEL_ROWS_VEC, (("fp32", "sum"),)),
             # fewer elements than ranks: one-element ranges, vectors spanning instances
             (24, 20, "ring", 0, 500, K.AR_KERNEL_ROWS_VEC, (("fp32", "sum"), ("int32", "sum"))),
             (24, 7, "ring", 0, 1001, K.AR_KERNEL_ROWS_VEC, (("fp32", "max"),)),
             (17, 16, "generalized", 0, 300, K.AR_KERNEL_ROWS_VEC, (("fp32", "sum"),)),
             # four elements per lane and one load per rank (up to 8 ranks), or
             # one element per lane and up to eight loads of four ranks each
             (4, 106, "ring", 0, 100, K.AR_KERNEL_ROWS_VEC, (("fp32", "sum"), ("int32", "max"))),
             (3, 106, "generalized", 0, 57, K.AR_KERNEL_ROWS_VEC, (("fp32", "avg"),)),
             (8, 64, "ring", 0, 129, K.AR_KERNEL_ROWS_VEC, (("fp32", "sum"), ("int32", "sum"))),
             (27, 90, "ring", 0, 213, K.AR_KERNEL_ROWS_VEC, (("fp32", "sum"),)),
             # 9-12 ranks with instances long enough that the range and map
             # table has more words than a single-wave workgroup has lanes
             (12, 500, "ring", 0, 60, K.AR_KERNEL_ROWS_VEC, (("fp32", "sum"), ("int32", "max"))),
             (10, 600, "generalized", 0, 45, K.AR_KERNEL_ROWS_VEC, (("fp32", "avg"),)),
             (11, 690, "ring", 0, 40, K.AR_KERNEL_ROWS_VEC, (("fp32", "max"),)),
             (24, 106, "generalized", 5, 500, K.AR_KERNEL_JIT, (("fp32", "sum"), ("int32", "max"), ("fp32", "avg"))),
             (24, 20_001, "generalized", 4, 1, K.AR_KERNEL_JIT, (("fp32", "sum"),)),
             (24, 106, "generalized", 1, 200, K.AR_KERNEL_STRIDED, (("fp32", "sum"),))]
    for i, (P, n, algo, knob, B, kern, types) in enumerate(cases):
        assert A.ar_kernel_of(A.make_call(P, n, "fp32", "sum", algo, knob, batch=B)) == kern, (P, n, algo, knob)
        for dtype, op in types:
            x = inputs.make(dtype, P, n * B, seed=300 + i)
            want = oracle.allreduce(x.reshape(P, B, n), algo, dtype, op, knob=knob, n=n)
            for mis in (False, True):
                got = gpu_allreduce(x, algo, dtype, op, knob, "fused", batch=B, misalign=mis)
                assert np.array_equal(bits(got.reshape(P, B, n)), bits(want)), (P, n, algo, knob, B, dtype, op, mis)
    x = inputs.make("fp32", 24, 106 * 100, seed=7)
    want = oracle.allreduce(x.reshape(24, 100, 106), "ring", "fp32", "sum", n=106)
    prev = A.ar_set_launch_blocks(3)
    try:
        got = gpu_allreduce(x, "ring", "fp32", "sum", 0, "fused", batch=100)
    finally:
        A.ar_set_launch_blocks(prev)
    assert np.array_equal(bits(got.reshape(24, 100, 106)), bits(want))
    # a grid smaller than the positions: every wave walks many of them
    x = inputs.make("fp32", 12, 50 * 3001, seed=8)
    want = oracle.allreduce(x.reshape(12, 3001, 50), "generalized", "fp32", "sum", n=50)
    prev = A.ar_set_launch_blocks(5)
    try:
        got = gpu_allreduce(x, "generalized", "fp32", "sum", 0, "fused", batch=3001)
    finally:
        A.ar_set_launch_blocks(prev)
    assert np.array_equal(bits(got.reshape(12, 3001, 50)), bits(want))
    # the same with at most 8 ranks (each lane evaluates its own vectors in
    # registers, the positions' loads alternating between two register sets)
    for P, n, B, algo, dtype, op, blocks in ((6, 106, 3001, "ring", "fp32", "sum", 5),
                                             (3, 106, 2999, "generalized", "int32", "max", 7),
                                             (5, 33, 4001, "ring", "fp32", "avg", 2)):
        x = inputs.make(dtype, P, n * B, seed=P + B)
        want = oracle.allreduce(x.reshape(P, B, n), algo, dtype, op, n=n)
        prev = A.ar_set_launch_blocks(blocks)
        try:
            got = gpu_allreduce(x, algo, dtype, op, 0, "fused", batch=B)
        finally:
            A.ar_set_launch_blocks(prev)
        assert np.array_equal(bits(got.reshape(P, B, n)), bits(want)), (P, n, B, algo, dtype, op)
    # the caller's events bracket the vector launch and the ragged tail's launch
    torch = torch_mod()
    x = inputs.make("fp32", 24, 106 * 39, seed=9)  # 4134 elements: 1033 vectors and 2 more
    bufs, keep = to_device(x, "fp32")
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    st = torch.cuda.current_stream()
    a.record(st)
    b.record(st)
    call = A.make_call(24, 106, "fp32", "sum", "ring", batch=39, start_event=a, stop_event=b)
    A.ar_allreduce_ex([t.data_ptr() for t in bufs], call, st)
    torch.cuda.synchronize()
    assert a.elapsed_time(b) > 0
    want = oracle.allreduce(x.reshape(24, 39, 106), "ring", "fp32", "sum", n=106).reshape(24, 39 * 106)
    assert np.array_equal(bits(from_device(bufs, "fp32")), bits(want))
    del keep


def test_auto_halves_run_the_oracle_choice():
    import allreduce_schedule_algorithms_amd as A
    from oracle import cost, schedules as sch
    m = A.ar_get_cost_model()
    for P in (5, 8):
        for n in (64, 1 << 16):
            x = inputs.make("fp32", P, n, seed=P * n)
            own = half_owner(n, P)
            a, r, _ = cost.select(P, n, "fp32", m["alpha"], m["beta"], m["gamma"], m["form"], coll="reduce_scatter")
            got = gpu_allreduce(x, "auto", "fp32", "sum", 0, "fused", collective="reduce_scatter")
            assert np.array_equal(bits(got[own, np.arange(n)]), bits(sch.reduce_scatter(x, a, "fp32", "sum"))), (P, n, a)


# --------------------------------------------------------------------------
# seeded random sweep over every option (the cases the CPU sweep draws)
# --------------------------------------------------------------------------
@pytest.mark.parametrize("seed", range(4))
def test_random_cases_on_gpu(seed):
    import allreduce_schedule_algorithms_amd as A
    from test_random_cpu import draw, oracle_result
    rng = np.random.default_rng(2000 + seed)
    for _ in range(25):
        coll, algo, knob, steps, factors, groups, P, n, batch, dtype, op = draw(rng)
        x = inputs.make(dtype, P, n * batch, seed=int(rng.integers(1 << 30)))
        want = oracle_result(coll, algo, knob, steps, factors, groups, P, n, batch, dtype, op, x)
        g = groups if algo == "ahc" else factors
        case = (coll, algo, knob, steps, factors, groups, P, n, batch, dtype, op)
        for ex in ("fused", "literal"):
            got = gpu_allreduce(x, algo, dtype, op, knob, ex, g, batch, collective=coll, steps=steps)
            if coll == "reduce_scatter":
                got = got.reshape(P, batch, n)[half_owner(n, P), :, np.arange(n)].T
            assert np.array_equal(bits(got), bits(want)), case + (ex,)


def test_long_work_split_over_launches():
    # with the per-launch workgroup limit lowered to 3, every executor cuts its
    # work into several launches; the results must not change
    import allreduce_schedule_algorithms_amd as A
    torch = torch_mod()
    cases = [  # (algo, knob, exec, P, n, misalign)
        ("rh_rd", 0, "fused", 8, 1 << 16, False),
        ("ring", 0, "fused", 5, 10_003, True),
        ("generalized", 2, "fused", 7, 50_001, False),   # several trees per range: staged kernel
        ("ring", 0, "literal", 5, 100_003, False),
        ("generalized", 3, "literal", 7, 20_000, True),
        ("direct", 0, "fused", 6, 10_003, False),        # vector path with an element tail
        ("direct", 0, "fused", 3, 10_000, True),         # element path
    ]
    prev = A.ar_set_launch_blocks(3)
    try:
        for algo, knob, ex, P, n, mis in cases:
            for dtype in ("fp32", "bf16"):
                x = inputs.make(dtype, P, n, seed=P * 31 + n)
                want = oracle.allreduce(x, algo, dtype, "sum", knob=knob)
                got = gpu_allreduce(x, algo, dtype, "sum", knob, ex, misalign=mis)
                assert np.array_equal(bits(got), bits(want)), (algo, knob, ex, P, n, mis, dtype)
        # the caller's events bracket the first and the last launch
        x = inputs.make("fp32", 8, 1 << 16, seed=5)
        bufs, keep = to_device(x, "fp32")
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        st = torch.cuda.current_stream()
        a.record(st)
        b.record(st)
        call = A.make_call(8, 1 << 16, "fp32", "sum", "rh_rd", start_event=a, stop_event=b)
        A.ar_allreduce_ex([t.data_ptr() for t in bufs], call, st)
        torch.cuda.synchronize()
        assert a.elapsed_time(b) > 0
        assert np.array_equal(bits(from_device(bufs, "fp32")), bits(oracle.allreduce(x, "rh_rd", "fp32", "sum")))
        del keep
    finally:
        A.ar_set_launch_blocks(prev)


def test_buffers_past_2_32_elements():
    # 2 ranks of 2^32 + 1000 fp32 (16 GiB each), one element off 16-byte
    # alignment: the element path needs 2^24 + 4 workgroups, one more than a
    # launch holds, and offsets pass 2^32 elements. Values are small integers
    # from a counter-based generator, so every sum is exact: sampled offsets are
    # checked against the oracle, and every offset against x0 + x1 (torch).
    import allreduce_schedule_algorithms_amd as A
    torch = torch_mod()
    P, n = 2, (1 << 32) + 1000
    cut = ((1 << 32) // 256 - 1) * 256  # first element of the second launch
    idx = np.unique(np.concatenate([
        inputs.sample_indices(n, P, count=4096),
        np.array([0, 1, 255, 256, cut - 1, cut, cut + 1, n // 2 - 1, n // 2, n // 2 + 1,
                  (1 << 31), (1 << 32) - 1, (1 << 32), n - 1], dtype=np.int64)]))
    xs = np.stack([inputs.counter_ints(p, idx).astype(np.float32) for p in range(P)])
    big = torch.empty((P, n + 8), dtype=torch.float32, device="cuda")
    rows = [big[p, 1: 1 + n] for p in range(P)]
    tidx = torch.from_numpy(idx).cuda()
    for algo, ex in (("ring", "fused"), ("direct", "fused"), ("ring", "literal")):
        for p in range(P):
            inputs.fill_counter_fp32(rows[p], p)
        call = A.make_call(P, n, "fp32", "sum", algo, 0, ex)
        A.ar_allreduce_ex([r.data_ptr() for r in rows], call, torch.cuda.current_stream())
        torch.cuda.synchronize()
        want = oracle.allreduce(xs, algo, "fp32", "sum", n=n, idx=idx)
        got = np.stack([r[tidx].cpu().numpy() for r in rows])
        assert np.array_equal(bits(got), bits(want)), (algo, ex)
        chunk = 1 << 27
        for s0 in range(0, n, chunk):
            e = torch.arange(s0, min(n, s0 + chunk), dtype=torch.int64, device="cuda")
            ref = (inputs.counter_ints(0, e) + inputs.counter_ints(1, e)).to(torch.float32)
            for r in rows:
                assert torch.equal(r[s0: s0 + e.numel()], ref), (algo, ex, s0)
    del rows, big


def test_calls_captured_in_a_hip_graph():
    # one-instance calls captured in a graph and replayed: every replay gives
    # the eager bits, with eager work (restoring the inputs) between replays
    import allreduce_schedule_algorithms_amd as A
    torch = torch_mod()
    n, B = 106, 40
    # fixed-shape kernels, and the compiled register DAG (several trees; a
    # latency-bound call over 12 ranks), launched as module kernels
    for P, algo, knob in ((6, "rd", 0), (6, "ring", 0), (6, "generalized", 1), (12, "rd", 0), (12, "generalized", 2)):
        if P == 12:
            assert A.ar_kernel_of(A.make_call(P, n, "fp32", "sum", algo, knob)) == A.Kernel.AR_KERNEL_JIT
        x = inputs.make("fp32", P, n * B, seed=B + knob + P)
        want = oracle.allreduce(x.reshape(P, B, n), algo, "fp32", "sum", knob=knob, n=n).reshape(P, B * n)
        bufs, keep = to_device(x, "fp32")
        pristine = [b.clone() for b in bufs]
        call = A.make_call(P, n, "fp32", "sum", algo, knob)
        st = torch.cuda.Stream()
        ptr_sets = [[b.data_ptr() + i * n * 4 for b in bufs] for i in range(B)]
        with torch.cuda.stream(st):
            for i in range(B):  # eager: builds the plan (no allocation may happen inside the capture)
                A.ar_allreduce_ex(ptr_sets[i], call, st)
        torch.cuda.synchronize()
        assert np.array_equal(bits(from_device(bufs, "fp32")), bits(want)), (algo, "eager")
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=st):
            for i in range(B):
                A.ar_allreduce_ex(ptr_sets[i], call, st)
        for rep in range(3):
            with torch.cuda.stream(st):
                for b, p0 in zip(bufs, pristine):
                    b.copy_(p0)
            torch.cuda.synchronize()
            g.replay()
            torch.cuda.synchronize()
            assert np.array_equal(bits(from_device(bufs, "fp32")), bits(want)), (algo, rep)
        del g, keep


def test_plans_survive_a_cleared_schedule_cache():
    # a plan built on the first call must stay valid after other specs have
    # pushed its schedule out of the schedule cache (more than 512 of them)
    import allreduce_schedule_algorithms_amd as A
    x = inputs.make("fp32", 5, 1000, seed=3)
    want = oracle.allreduce(x, "ring", "fp32", "sum")
    for ex in ("fused", "literal"):
        assert np.array_equal(bits(gpu_allreduce(x, "ring", "fp32", "sum", 0, ex)), bits(want))
    for n in range(1, 530):
        A.ar_workspace_bytes(A.make_call(3, n, "fp32", "sum", "ring", 0, "literal"))
    for ex in ("fused", "literal"):
        assert np.array_equal(bits(gpu_allreduce(x, "ring", "fp32", "sum", 0, ex)), bits(want))
    # more than 256 plans (distinct sizes) clear the plan cache: the plans a
    # later call builds again must give the same bits
    torch = torch_mod()
    bufs = [torch.zeros(300, dtype=torch.float32, device="cuda") for _ in range(3)]
    for n in range(1, 280):
        A.ar_allreduce([b.data_ptr() for b in bufs], 3, n, "fp32", "sum", "ring")
    torch.cuda.synchronize()
    for ex in ("fused", "literal"):
        assert np.array_equal(bits(gpu_allreduce(x, "ring", "fp32", "sum", 0, ex)), bits(want))


def test_many_ranks_ragged_ranges_in_sized_items():
    # programs of many ranges over many ranks on ragged sizes: the program-driven
    # replay sizes its items to whole rounds of workgroups over the compute
    # units (items of 16-vector multiples below 256, partial vectors at every
    # range end); every element against the oracle
    import allreduce_schedule_algorithms_amd as A
    cases = [(40, 30011, "bf16", "sum", "ring", 0), (70, 50001, "fp32", "max", "generalized", 0),
             (100, 123457, "bf16", "avg", "ahc", 0), (150, 400003, "bf16", "sum", "ring", 0),
             (63, 200001, "int32", "sum", "generalized", 0), (129, 99991, "fp32", "sum", "ring", 0)]
    for i, (P, n, dtype, op, algo, r) in enumerate(cases):
        g = groups_for(algo, P)
        assert A.ar_kernel_of(A.make_call(P, n, dtype, op, algo, r, groups=g)) == A.Kernel.AR_KERNEL_REPLAY, (P, algo)
        x = inputs.make(dtype, P, n, seed=900 + i)
        want = oracle.allreduce(x, algo, dtype, op, knob=r, groups=g)
        got = gpu_allreduce(x, algo, dtype, op, r, "fused", g)
        assert np.array_equal(bits(got), bits(want)), (P, n, dtype, op, algo)


def test_random_large_cases_on_gpu():
    # larger random cases than the 2-16 rank draws above: 9-192 ranks, up to
    # 3 x 10^5 elements, one- and many-range schedules, aligned and unaligned
    # buffers, so that the round-sized items, the masked range ends, the
    # compiled kernels and their element paths all run; every element against
    # the oracle
    import allreduce_schedule_algorithms_amd as A
    rng = np.random.default_rng(4242)
    kernels = set()
    for _ in range(30):
        P = int(rng.choice([9, 12, 17, 24, 33, 40, 63, 100, 127, 192]))
        algo = str(rng.choice(["ring", "rh_rd", "rd", "binomial", "generalized", "ahc", "direct", "chain"]))
        knob = int(rng.integers(1, 9)) if algo == "chain" else 0
        if algo == "generalized" and P <= 24:
            knob = int(rng.integers(0, nu.ceil_log2(P) + 1))
        n = int(rng.integers(1000, 300_000 if P <= 64 else 100_000))
        dtype = str(rng.choice(["int32", "fp32", "bf16"]))
        op = str(rng.choice(["sum", "max"] + (["avg"] if dtype != "int32" else [])))
        mis = bool(rng.random() < 0.25)
        g = groups_for(algo, P)
        kernels.add(A.ar_kernel_of(A.make_call(P, n, dtype, op, algo, knob, groups=g)).name)
        x = inputs.make(dtype, P, n, seed=int(rng.integers(1 << 30)))
        want = oracle.allreduce(x, algo, dtype, op, knob=knob, groups=g)
        got = gpu_allreduce(x, algo, dtype, op, knob, "fused", g, misalign=mis)
        assert np.array_equal(bits(got), bits(want)), (P, n, algo, knob, dtype, op, mis)
    assert len(kernels) >= 4, kernels
