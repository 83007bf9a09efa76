"""Host-side checks of the library's schedule layer (no GPU needed).

The exported step tables and fused programs are executed by the generic
interpreters in table_interp.py and must give exactly the oracle's bits; the
library's own checks, step counts, traffic and cost report are compared with
the pages' facts and with the oracle's independent counters.
"""
import math
import os
import re
import subprocess

import numpy as np
import pytest

import allreduce_schedule_algorithms_amd as A
import oracle
from oracle import cost as ocost, numerics as nu
from synth import inputs
from table_interp import run_fused, run_table

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ALGOS = ("direct", "ring", "rh_rd", "rd", "binomial", "generalized", "generalized_xor", "ahc")


def knobs(algo, P):
    return range(nu.ceil_log2(P) + 1) if algo.startswith("generalized") else [0]


def groups_for(algo, P):
    if algo != "ahc":
        return None
    return [P] if P < 3 else [P // 3 + 1, P - (P // 3 + 1)]


def build(algo, P, n, dtype="fp32", op="sum", knob=0, groups=None, batch=1, exec="fused"):
    return A.ar_schedule_build(A.make_call(P, n, dtype, op, algo, knob, exec=exec, batch=batch,
                                           groups=groups if groups is not None else groups_for(algo, P)))


def as_bits(a):
    a = np.asarray(a)
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


@pytest.mark.parametrize("algo", ALGOS)
@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
def test_table_and_fused_program_match_oracle(algo, dtype):
    for P in (2, 3, 5, 7, 8, 12):
        if algo == "generalized_xor" and P & (P - 1):
            continue
        for n in (1, 6, 37, 211):
            for r in knobs(algo, P):
                for op in ("sum", "max"):
                    x = inputs.make(dtype, P, n, seed=P * 31 + n)
                    want = oracle.allreduce(x, algo, dtype, op, knob=r, groups=groups_for(algo, P))
                    s = build(algo, P, n, dtype, op, r)
                    got = run_table(x, s.export(), dtype, op, n)
                    assert np.array_equal(as_bits(got), as_bits(want)), (algo, P, n, r, op)
                    st, ln, off, words = s.fused_export()
                    fz = run_fused(x, st, ln, off, words, dtype, op, n)
                    assert np.array_equal(as_bits(fz), as_bits(want)), (algo, P, n, r, op, "fused")


@pytest.mark.parametrize("algo", ["ring", "rd", "binomial", "generalized", "ahc"])
def test_batched_table_and_program(algo):
    P, n, B = 6, 53, 5
    for r in knobs(algo, P):
        x = inputs.make("fp32", P, B * n, seed=9, dist="uniform_pm1")
        want = oracle.allreduce(x.reshape(P, B, n), algo, "fp32", "sum", knob=r, groups=groups_for(algo, P), n=n)
        want = want.reshape(P, B * n)
        s = build(algo, P, n, "fp32", "sum", r, batch=B)
        assert np.array_equal(run_table(x, s.export(), "fp32", "sum", n, batch=B), want)
        st, ln, off, words = s.fused_export()
        assert np.array_equal(run_fused(x, st, ln, off, words, "fp32", "sum", n, batch=B), want)


def test_config_tables_cpu():
    # 5-rank 4096-element int32 ring: 8 steps, all ranks equal the brute force
    x = inputs.workload("ring_int32")
    s = build("ring", 5, 4096, "int32")
    assert s.info().steps == 8
    got = run_table(x, s.export(), "int32", "sum", 4096)
    assert np.array_equal(got, np.broadcast_to(nu.brute_force(x, "int32", "sum"), got.shape))
    # AHC (64, 128) at a reduced length: 256 chunks, 256 steps
    n = 256 * 8
    xb = inputs.make("bf16", 192, n, seed=0)
    s = build("ahc", 192, n, "bf16", "sum", groups=[64, 128])
    inf = s.info()
    assert inf.steps == 256 and inf.atoms == 256
    want = oracle.allreduce(xb, "ahc", "bf16", "sum", groups=[64, 128])
    assert np.array_equal(run_table(xb, s.export(), "bf16", "sum", n), want)
    st, ln, off, words = s.fused_export()
    assert np.array_equal(run_fused(xb, st, ln, off, words, "bf16", "sum", n), want)


# --------------------------------------------------------------------------
# step counts, ports, traffic
# --------------------------------------------------------------------------
def test_step_counts_match_oracle():
    for algo in ALGOS:
        for P in (2, 3, 5, 6, 7, 8, 12, 16, 24):
            if algo == "generalized_xor" and P & (P - 1):
                continue
            for r in knobs(algo, P):
                _, st = oracle.allreduce(np.zeros((P, P), np.int32), algo, "int32", "sum", knob=r,
                                         groups=groups_for(algo, P), return_stats=True)
                assert build(algo, P, 4 * P, knob=r).info().steps == st["steps"], (algo, P, r)


def test_per_step_traffic_matches_oracle():
    # the oracle's simulator counts every element sent / combined per rank and step
    for algo in ("direct", "ring", "rh_rd", "rd", "binomial", "ahc"):
        for P in (3, 5, 8, 12):
            n = 97
            _, st = oracle.allreduce(np.zeros((P, n), np.int32), algo, "int32", "sum",
                                     groups=groups_for(algo, P), return_stats=True)
            s = build(algo, P, n)
            sent, recv, red = s.cost_steps(P)
            assert np.array_equal(sent, st["sent"]), (algo, P)
            assert np.array_equal(recv, st["recv"]), (algo, P)
            assert np.array_equal(red, st["reduced"]), (algo, P)


def test_generalized_traffic_matches_oracle_counts():
    for P in (5, 6, 7, 12, 13):
        L = nu.ceil_log2(P)
        for r in range(L + 1):
            _, st = oracle.allreduce(np.zeros((P, P), np.int32), "generalized", "int32", "sum", knob=r,
                                     return_stats=True)
            s = build("generalized", P, P, knob=r)  # one element per part
            sent, _, red = s.cost_steps(P)
            # every rank sends the same number of parts in every step
            assert (sent == sent[:, :1]).all()
            assert list(sent[:L, 0]) == st["reduction_sent_parts"]
            assert list(red[:L, 0]) == st["reduction_reduced_parts"]
            assert list(sent[L:, 0]) == st["distribution_sent_parts"]


def test_single_port_flags():
    for algo in ("direct", "ring", "rh_rd", "rd", "binomial", "generalized", "generalized_xor"):
        for P in (4, 5, 8, 12):
            if algo == "generalized_xor" and P & (P - 1):
                continue
            for r in knobs(algo, P):
                assert build(algo, P, 64, knob=r).info().single_port == 1, (algo, P, r)
    # AHC phase 2: a rank may own pieces paired with several owners
    assert build("ahc", 192, 4096, groups=[64, 128]).info().single_port == 0


def test_ring_traffic_formula():
    # each rank sends 2(P-1)n/P elements (blog page, "The ring algorithm")
    for P in (4, 8):
        n = 64 * P
        c = build("ring", P, n).cost()
        assert c.max_rank_sent == 2 * (P - 1) * n // P
        assert c.sent_total == 2 * (P - 1) * n


def test_in_place_slots():
    # bandwidth-optimal schedules run in the caller's buffers; bf16 partials use one fp32 slot
    for algo in ("ring", "rh_rd", "rd", "binomial", "direct"):
        assert build(algo, 8, 64, "fp32").info().slots == 1
        assert build(algo, 8, 64, "bf16").info().slots == 2
    assert build("ahc", 192, 4096, "bf16", groups=[64, 128]).info().slots == 2
    # the generalized algorithm keeps q* and q' apart (paper, latency-optimal section)
    assert build("generalized", 7, 7, knob=1).info().slots == 2


def test_fused_program_shape():
    for P in (5, 7, 8):
        inf = build("ring", P, 10 * P).info()
        assert inf.ranges == P and inf.max_trees == 1 and inf.max_need == 2
    inf = build("rh_rd", 8, 64).info()
    assert inf.ranges == 1 and inf.max_need == 4
    inf = build("generalized", 7, 70, knob=3).info()
    assert inf.max_trees == 7
    # AHC (64, 128): 128 pieces; the two sub-pieces of a piece differ only in the order of
    # the two group sums, which commutes, so each piece is one range
    inf = build("ahc", 192, 4096, "bf16", groups=[64, 128]).info()
    assert inf.ranges == 128 and inf.max_trees == 1 and inf.max_leaves == 192 and inf.max_need == 3


# --------------------------------------------------------------------------
# table checker: corrupted tables are rejected
# --------------------------------------------------------------------------
def test_table_check_accepts_exports():
    for algo in ALGOS:
        for P in (5, 8):
            if algo == "generalized_xor" and P & (P - 1):
                continue
            for r in knobs(algo, P):
                ops = build(algo, P, 40, "bf16", knob=r).export()
                A.ar_table_check(P, 40, "bf16", ops)


def test_table_check_rejects_dropped_op():
    ops = build("ring", 5, 50).export()
    bad = ops[:3] + ops[4:]
    with pytest.raises(A.ArError, match="complete"):
        A.ar_table_check(5, 50, "fp32", bad)


def test_table_check_rejects_duplicate_write():
    ops = build("ring", 5, 50).export()
    dup = A._ar.ar_oprec()
    for f, _ in A._ar.ar_oprec._fields_:
        setattr(dup, f, getattr(ops[0], f))
    dup.src_rank = (ops[0].src_rank + 2) % 5
    bad = ops[:1] + [dup] + ops[1:]
    with pytest.raises(A.ArError, match="overlap"):
        A.ar_table_check(5, 50, "fp32", bad)


def test_table_check_rejects_same_step_read_after_write():
    # moving the second reduce-scatter step into the first breaks snapshot semantics
    ops = build("ring", 5, 50).export()
    for o in ops:
        if o.step == 1:
            o.step = 0
    ops.sort(key=lambda o: o.step)
    with pytest.raises(A.ArError):
        A.ar_table_check(5, 50, "fp32", ops)


def test_table_check_rejects_bf16_partial_in_user_buffer():
    ops = build("ring", 5, 50, "bf16").export()
    for o in ops:
        if o.kind == 0 and o.dst_slot != 0:
            o.dst_slot = 0
            break
    with pytest.raises(A.ArError):
        A.ar_table_check(5, 50, "bf16", ops)


# --------------------------------------------------------------------------
# cost report
# --------------------------------------------------------------------------
def test_cost_closed_forms():
    alpha, beta, gamma = 2e-6, 1e-10, 3e-11
    for P in (4, 8, 16):
        n = 64 * P
        for algo, r in (("ring", 0), ("rh_rd", 0), ("generalized", 0), ("generalized_xor", 0)):
            c = build(algo, P, n, knob=r).cost(alpha, beta, gamma)
            assert c.predicted_seconds == pytest.approx(c.closed_form_seconds, rel=1e-12), (algo, P)
        c = build("rd", P, n).cost(alpha, beta, gamma)
        assert c.predicted_seconds == pytest.approx(c.closed_form_seconds, rel=1e-12)
        c = build("binomial", P, n).cost(alpha, beta, gamma)
        assert c.predicted_seconds == pytest.approx(c.closed_form_seconds, rel=1e-12)
    # the oracle's prose forms agree with the library's closed forms
    P, n = 7, 7 * 100
    m = n * 4
    for r in range(3):
        c = build("generalized", P, n, knob=r).cost(alpha, beta, gamma)
        assert c.closed_form_seconds == pytest.approx(ocost.intermediate_time(P, m, r, alpha, beta, gamma))
    c = build("ring", P, n).cost(alpha, beta, gamma)
    assert c.closed_form_seconds == pytest.approx(ocost.ring_time(P, m, alpha, beta, gamma))
    assert math.isnan(build("ahc", 5, 60, groups=[2, 3]).cost(alpha, beta, gamma).closed_form_seconds)


def test_cost_bytes():
    c = build("ring", 8, 1 << 12).cost()
    n = 1 << 12
    assert c.essential_bytes == 2 * 8 * n * 4
    assert c.fused_hbm_bytes == c.essential_bytes
    assert c.literal_hbm_bytes == 5 * 7 * n * 4  # 3 accesses per reduced, 2 per copied element
    c = build("generalized", 7, 7 * 64, knob=3).cost()
    assert c.fused_hbm_bytes > c.essential_bytes  # seven distinct trees reload their leaves


# --------------------------------------------------------------------------
# the C ABI: every declared symbol is exported; host-side validation
# --------------------------------------------------------------------------
def declared_functions():
    with open(os.path.join(ROOT, "include", "ar.h")) as f:
        text = f.read()
    return sorted(set(re.findall(r"^\s*(?:const\s+)?[a-z_0-9]+\*?\s+\*?(ar_[a-z_]+)\s*\(", text, re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert len(names) >= 15
    out = subprocess.run(["nm", "-D", "--defined-only", A._ar.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ar_[a-z_]+)\b", out))
    for nm in names:
        assert nm in exported, nm
        assert hasattr(A._ar.lib, nm)
        assert nm in A._ar.SIGNATURES


FAKE = [0x1000 * (i + 1) for i in range(256)]


@pytest.mark.parametrize("kw,match", [
    (dict(P=0), "P must"), (dict(P=257), "P must"), (dict(n=-1), "n must"), (dict(dtype=7), "dtype"),
    (dict(op=5), "op"), (dict(algo=11), "algorithm"), (dict(algo="generalized", knob=4), "knob"),
    (dict(algo="generalized", knob=-2), "knob"), (dict(algo="generalized_xor", P=6), "power of two"),
    (dict(algo="ahc", groups=[2, 2]), "sum to P"), (dict(algo="ahc", groups=None), "group"),
    (dict(algo="ahc", groups=[5, 0]), "group sizes"), (dict(exec=9), "exec"),
    (dict(collective=3), "collective"), (dict(op="avg", dtype="int32"), "avg"),
    (dict(algo="rd", collective="reduce_scatter"), "reduce-scatter"),
    (dict(algo="rh_rd", P=6, collective="all_gather"), "power of two"),
    (dict(algo="generalized", knob=1, collective="reduce_scatter"), "r = 0"),
    (dict(algo="ring", steps=4), "steps"), (dict(algo="generalized", steps=2), "steps"),
    (dict(algo="generalized", steps=5), "steps"), (dict(algo="generalized", groups=[2, 2]), "product"),
    (dict(algo="chain", knob=0), "pieces"), (dict(algo="chain", knob=5000), "pieces"),
])
def test_invalid_arguments_rejected_before_device_work(kw, match):
    args = dict(P=5, n=100, dtype="fp32", op="sum", algo="ring", knob=0, exec="fused", groups=None,
                collective="allreduce", steps=0)
    args.update(kw)
    call = A.make_call(args["P"], args["n"], args["dtype"], args["op"], args["algo"], args["knob"],
                       args["exec"], groups=args["groups"], steps=args["steps"])
    call.collective = args["collective"] if isinstance(args["collective"], int) else \
        int(A.COLLECTIVES[args["collective"]])
    with pytest.raises(A.ArError, match=match) as e:
        A.ar_allreduce_ex(FAKE[: max(args["P"], 1)], call)
    assert e.value.status == A.Status.AR_INVALID_ARGUMENT


def test_null_and_duplicate_buffers_rejected():
    with pytest.raises(A.ArError, match="NULL"):
        A.ar_allreduce([FAKE[0], 0, FAKE[2]], 3, 10, "fp32", "sum", "ring")
    with pytest.raises(A.ArError, match="share"):
        A.ar_allreduce([FAKE[0], FAKE[1], FAKE[0]], 3, 10, "fp32", "sum", "ring")
    with pytest.raises(A.ArError, match="ar_allreduce_ex"):
        A.ar_allreduce(FAKE[:3], 3, 10, "fp32", "sum", "ahc")


def test_half_entry_points_validate_before_device_work():
    with pytest.raises(A.ArError, match="reduce-scatter"):
        A.ar_reduce_scatter(FAKE[:5], 5, 100, "fp32", "sum", "binomial")
    with pytest.raises(A.ArError, match="AHC"):
        A.ar_all_gather(FAKE[:5], 5, 100, "fp32", "ahc")
    with pytest.raises(A.ArError, match="share"):
        A.ar_all_gather([FAKE[0], FAKE[0]], 2, 100, "fp32", "ring")
    # nothing to move: valid, no device work
    A.ar_reduce_scatter(FAKE[:1], 1, 100, "bf16", "avg", "ring")
    A.ar_all_gather(FAKE[:4], 4, 0, "int32", "generalized")
    with pytest.raises(A.ArError, match="NULL"):
        A._ar._check(A._ar.lib.ar_table_check_ex(None, None, 0, None))


def test_trivial_calls_do_no_device_work():
    # one rank or empty buffers: valid, nothing to combine, no HIP call is made
    A.ar_allreduce(FAKE[:1], 1, 1000, "fp32", "sum", "ring")
    A.ar_allreduce(FAKE[:4], 4, 0, "bf16", "max", "rd")


def test_workspace_query():
    lit = A.make_call(8, 1024, "bf16", "sum", "ring", exec="literal")
    assert A.ar_workspace_bytes(lit) == 8 * 1024 * 4  # one fp32 slot per rank
    assert A.ar_workspace_bytes(A.make_call(8, 1024, "bf16", "sum", "ring")) == 0
    assert A.ar_workspace_bytes(A.make_call(8, 1024, "fp32", "sum", "ring", exec="literal")) == 0
    # ranges with more result trees than the register replays keep run the
    # compiled register DAG (or, over more ranks, the DAG replay): no workspace
    big = A.make_call(13, 1000, "fp32", "sum", "generalized", 4, steps=4)
    assert A.ar_schedule_build(big).info().max_trees > 8
    assert A.ar_kernel_of(big) == A.Kernel.AR_KERNEL_JIT
    assert A.ar_workspace_bytes(big) == 0
    bigger = A.make_call(63, 1000, "fp32", "sum", "generalized", 6)
    assert A.ar_kernel_of(bigger) == A.Kernel.AR_KERNEL_DAG
    assert A.ar_workspace_bytes(bigger) == 0
    lit = A.make_call(13, 1000, "fp32", "sum", "generalized", 4, "literal", steps=4)
    assert A.ar_workspace_bytes(lit) > 0
    # a DAG whose values exceed a workgroup's LDS (255 ranks, r = 8) runs the
    # literal steps and needs their workspace
    huge = A.make_call(255, 600, "fp32", "sum", "generalized", 8)
    assert A.ar_kernel_of(huge) == A.Kernel.AR_KERNEL_LITERAL
    lit = A.make_call(255, 600, "fp32", "sum", "generalized", 8, "literal")
    assert A.ar_workspace_bytes(huge) == A.ar_workspace_bytes(lit) > 0


def test_kernel_choice():
    # which kernel family a call runs: the host's choice, by schedule shape and size
    K = A.Kernel
    cases = [
        (dict(P=8, n=1 << 20, algo="rh_rd"), K.AR_KERNEL_FIXED_BALANCED),
        (dict(P=4, n=4099, algo="rd"), K.AR_KERNEL_FIXED_BALANCED),
        (dict(P=8, n=1 << 20, algo="ring"), K.AR_KERNEL_FIXED_CHAIN),
        (dict(P=5, n=77, algo="chain", knob=3), K.AR_KERNEL_FIXED_CHAIN),
        (dict(P=7, n=1 << 24, algo="ring", collective="all_gather"), K.AR_KERNEL_FIXED_CHAIN),
        (dict(P=7, n=1 << 24, algo="generalized"), K.AR_KERNEL_FIXED_STACK),
        (dict(P=6, n=1000, algo="binomial"), K.AR_KERNEL_FIXED_STACK),
        (dict(P=7, n=1 << 24, algo="generalized", knob=3), K.AR_KERNEL_JIT),
        (dict(P=7, n=1 << 24, algo="generalized", knob=1), K.AR_KERNEL_JIT),
        (dict(P=7, n=1 << 20, algo="generalized", knob=2, dtype="bf16"), K.AR_KERNEL_JIT),
        (dict(P=12, n=4099, algo="generalized", knob=2), K.AR_KERNEL_JIT),
        (dict(P=24, n=106, algo="generalized", knob=5, batch=10_000), K.AR_KERNEL_JIT),
        # bf16 values take two registers each: 24 live leaves exceed the budget
        (dict(P=24, n=106, algo="generalized", knob=5, batch=10_000, dtype="bf16"), K.AR_KERNEL_DAG),
        (dict(P=24, n=106, algo="generalized", knob=5, batch=30), K.AR_KERNEL_JIT),
        (dict(P=24, n=106, algo="rd"), K.AR_KERNEL_JIT),  # latency-bound over more than 8 ranks
        (dict(P=24, n=106, algo="binomial"), K.AR_KERNEL_JIT),
        (dict(P=24, n=106, algo="generalized"), K.AR_KERNEL_DAG),  # 24 ranges: more than the compiled form takes
        (dict(P=127, n=106, algo="generalized"), K.AR_KERNEL_DAG),
        (dict(P=24, n=106, algo="ring"), K.AR_KERNEL_REPLAY),  # a chain: one level per rank
        (dict(P=12, n=106, algo="rd"), K.AR_KERNEL_JIT),
        (dict(P=12, n=5000, algo="rd"), K.AR_KERNEL_REPLAY),
        (dict(P=192, n=1 << 20, dtype="bf16", algo="ahc", groups=[64, 128]), K.AR_KERNEL_REPLAY),
        (dict(P=24, n=106, algo="rd", batch=10_000), K.AR_KERNEL_REPLAY),
        (dict(P=24, n=106, algo="generalized", batch=10_000), K.AR_KERNEL_ROWS_VEC),
        (dict(P=24, n=106, algo="ring", batch=10_000), K.AR_KERNEL_ROWS_VEC),
        (dict(P=24, n=106, algo="ring", batch=10_000, dtype="bf16"), K.AR_KERNEL_ROWS),
        (dict(P=24, n=106, algo="ring", batch=30), K.AR_KERNEL_ROWS),
        (dict(P=24, n=106, algo="generalized", knob=1, batch=10_000), K.AR_KERNEL_STRIDED),
        (dict(P=8, n=1 << 20, algo="direct"), K.AR_KERNEL_DIRECT),
        (dict(P=8, n=1 << 20, algo="direct", exec="replay"), K.AR_KERNEL_FIXED_CHAIN),
        (dict(P=8, n=1 << 20, algo="direct", collective="reduce_scatter"), K.AR_KERNEL_FIXED_CHAIN),
        (dict(P=8, n=1 << 20, algo="ring", exec="literal"), K.AR_KERNEL_LITERAL),
        (dict(P=13, n=1000, algo="generalized", knob=4, steps=4), K.AR_KERNEL_JIT),  # more than 8 trees
        (dict(P=17, n=1000, algo="generalized", knob=4), K.AR_KERNEL_DAG),  # more ranks than the compiled form
        (dict(P=127, n=106, algo="generalized", knob=7), K.AR_KERNEL_DAG),
        (dict(P=127, n=1 << 16, algo="generalized", knob=4), K.AR_KERNEL_DAG),
        (dict(P=63, n=106, algo="generalized", knob=6), K.AR_KERNEL_DAG),
        (dict(P=100, n=106, algo="generalized", knob=7), K.AR_KERNEL_DAG),
        (dict(P=255, n=600, algo="generalized", knob=8), K.AR_KERNEL_LITERAL),  # its DAG exceeds the LDS
        (dict(P=8, n=1 << 20, algo="rh_rd", exec="dag"), K.AR_KERNEL_DAG),
        (dict(P=8, n=1 << 20, algo="direct", exec="dag"), K.AR_KERNEL_DAG),
        (dict(P=1, n=10, algo="ring"), K.AR_KERNEL_NONE),
        (dict(P=5, n=0, algo="ring"), K.AR_KERNEL_NONE),
    ]
    for kw, want in cases:
        kw = dict(kw)
        P, n = kw.pop("P"), kw.pop("n")
        dtype, algo, knob = kw.pop("dtype", "fp32"), kw.pop("algo"), kw.pop("knob", 0)
        ex = kw.pop("exec", "fused")
        got = A.ar_kernel_of(A.make_call(P, n, dtype, "sum", algo, knob, ex, **kw))
        assert got == want, (P, n, algo, knob, ex, kw, got)
    with pytest.raises(A.ArError):
        A.ar_kernel_of(A.make_call(6, 100, "fp32", "sum", "generalized_xor"))  # Z_2^k needs a power of two


def test_launch_block_limit_setter():
    top = (1 << 32) // 256 - 1
    prev = A.ar_set_launch_blocks(5)
    try:
        assert prev == top  # the default is the dispatch limit
        assert A.ar_set_launch_blocks(7) == 5
        for bad in (0, -1, top + 1):
            with pytest.raises(A.ArError) as e:
                A.ar_set_launch_blocks(bad)
            assert e.value.status == A.Status.AR_INVALID_ARGUMENT
        assert A.ar_set_launch_blocks(top) == 7  # a rejected value changes nothing
    finally:
        A.ar_set_launch_blocks(prev)


def test_status_strings():
    assert A.ar_status_string(0) == "AR_OK"
    assert A.ar_status_string(3) == "AR_WORKSPACE_TOO_SMALL"


def test_probe_library_exports_every_declared_symbol():
    # the measurement library (memory-traffic ceilings) that bench.py loads
    from allreduce_schedule_algorithms_amd import probe
    with open(os.path.join(ROOT, "include", "ar_probe.h")) as f:
        names = sorted(set(re.findall(r"^\s*[a-z_0-9]+\s+(ar_[a-z_]+)\s*\(", f.read(), re.M)))
    assert names == ["ar_probe_last_hip_error", "ar_probe_stream"]
    out = subprocess.run(["nm", "-D", "--defined-only", probe.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (ar_[a-z_]+)\b", out))
    for nm in names:
        assert nm in exported, nm
        assert nm in probe.SIGNATURES
