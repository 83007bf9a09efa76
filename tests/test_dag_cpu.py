"""The DAG form of the fused program (what AR_KERNEL_DAG runs), interpreted on
the CPU: every level's combinations independent (checked, and run in reverse
order), one program per range or one shared program with per-range renamings,
and the results bit-identical to the oracle's replay of the schedule."""
import numpy as np
import pytest

import allreduce_schedule_algorithms_amd as A
import oracle
from oracle import numerics as nu
from synth import inputs
from table_interp import dag_parse, run_dag


def bits(a):
    a = np.asarray(a)
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


def dag_result(x, algo, dtype, op, knob, n, batch=1, groups=None, steps=0):
    P = x.shape[0]
    s = A.ar_schedule_build(A.make_call(P, n, dtype, op, algo, knob, batch=batch, groups=groups, steps=steps))
    st, ln, _, _ = s.fused_export()
    shared, offs, maps, words = s.dag_export()
    return run_dag(x, st, ln, shared, offs, maps, words, dtype, op, n, batch)


@pytest.mark.parametrize("dtype", ["int32", "fp32", "bf16"])
def test_dag_matches_oracle_generalized(dtype):
    for P in (3, 5, 6, 7, 8, 12, 13):
        for n in (1, 37, 211):
            for r in range(nu.ceil_log2(P) + 1):
                x = inputs.make(dtype, P, n, seed=P * 5 + n + r)
                for op in ("sum", "max") + (("avg",) if dtype != "int32" else ()):
                    want = oracle.allreduce(x, "generalized", dtype, op, knob=r)
                    got = dag_result(x, "generalized", dtype, op, r, n)
                    assert np.array_equal(bits(got), bits(want)), (P, n, r, op)


@pytest.mark.parametrize("algo", ["ring", "rh_rd", "rd", "binomial", "direct", "generalized_xor", "ahc"])
def test_dag_matches_oracle_single_tree_schedules(algo):
    # one tree per range: the DAG is the tree itself, levels by depth
    for P in (4, 6, 8):
        if algo == "generalized_xor" and P & (P - 1):
            continue
        groups = [P // 2, P - P // 2] if algo == "ahc" else None
        x = inputs.make("fp32", P, 97, seed=P)
        want = oracle.allreduce(x, algo, "fp32", "sum", groups=groups)
        assert np.array_equal(bits(dag_result(x, algo, "fp32", "sum", 0, 97, groups=groups)), bits(want)), (algo, P)


def test_dag_large_rank_counts():
    # the paper's experiment size: P = 127 (and 63, 100), every r, one element per part
    for P in (63, 100, 127):
        L = nu.ceil_log2(P)
        x = inputs.make("fp32", P, 106, seed=P, dist="uniform_pm1")
        for r in range(L + 1):
            want = oracle.allreduce(x, "generalized", "fp32", "sum", knob=r)
            assert np.array_equal(bits(dag_result(x, "generalized", "fp32", "sum", r, 106)), bits(want)), (P, r)


def test_dag_batched_steps_and_groups():
    P, n, B = 12, 53, 4
    x = inputs.make("fp32", P, n * B, seed=7)
    for r in (1, 3, 4):
        want = oracle.allreduce(x.reshape(P, B, n), "generalized", "fp32", "sum", knob=r, n=n).reshape(P, B * n)
        assert np.array_equal(bits(dag_result(x, "generalized", "fp32", "sum", r, n, batch=B)), bits(want)), r
    x = inputs.make("fp32", P, 60, seed=8)
    for r in (0, 2, 5):
        want = oracle.allreduce(x, "generalized", "fp32", "sum", knob=r, steps=5)
        assert np.array_equal(bits(dag_result(x, "generalized", "fp32", "sum", r, 60, steps=5)), bits(want)), r
    for f in ((2, 6), (3, 4), (2, 2, 3)):
        for r in (1, 2):
            want = oracle.allreduce(x, "generalized", "fp32", "sum", knob=r, factors=f)
            got = dag_result(x, "generalized", "fp32", "sum", r, 60, groups=list(f))
            assert np.array_equal(bits(got), bits(want)), (f, r)


def test_dag_evaluates_each_distinct_combination_once():
    # generalized over Z_7, latency-optimal (r = 3): the seven result trees of a
    # part share their sub-trees; the reduction phase combines (2L - 2) P parts
    # per rank in all (prose pin of the latency-optimal section), and the DAG
    # holds exactly those distinct combinations per element offset
    s = A.ar_schedule_build(A.make_call(7, 7, "fp32", "sum", "generalized", 3))
    shared, offs, maps, words = s.dag_export()
    S, leaves, lv, ins, outs = dag_parse(words, 0)
    assert len(ins) == (2 * 3 - 2) * 7 == 28
    assert len(lv) - 1 == 3 and sorted(leaves) == list(range(7))
    assert sorted(q for _, q in outs) == list(range(7))
    # P = 127, r = 7: (2L - 2) P = 1524 distinct combinations per element
    s = A.ar_schedule_build(A.make_call(127, 127, "fp32", "sum", "generalized", 7))
    _, _, _, words = s.dag_export()
    assert dag_parse(words, 0)[3].__len__() == 12 * 127


def test_dag_hazard_check_catches_a_planted_reuse():
    # a program whose level writes a slot another combination of the same level
    # reads must be rejected by the checker the interpreter runs
    from table_interp import dag_hazards
    s = A.ar_schedule_build(A.make_call(7, 7, "fp32", "sum", "generalized", 3))
    prog = list(dag_parse(s.dag_export()[3], 0))
    ins = list(prog[3])
    lv = prog[2]
    d0, a0, b0 = ins[lv[0]]
    d1, a1, b1 = ins[lv[0] + 1]
    ins[lv[0]] = (a1, a0, b0)  # the first combination overwrites an operand of the second
    prog[3] = ins
    with pytest.raises(AssertionError):
        dag_hazards(tuple(prog))
