"""Seeded random sweep over every option at once (CPU): collective, op, dtype,
schedule, knob, reduction steps, group factors, batch and ragged sizes. The
library's exported table and fused program, run by the generic interpreters,
must give the oracle's bits for each drawn case."""
import numpy as np
import pytest

import allreduce_schedule_algorithms_amd as A
from oracle import numerics as nu, schedules as sch
from synth import inputs
from table_interp import run_fused, run_table


def factorizations(P):
    out = [None]
    for a in range(2, P):
        if P % a == 0 and P // a >= 2:
            out.append([a, P // a])
    return out


def draw(rng):
    """One random valid case: (collective, algo, knob, steps, factors, groups, P, n, batch, dtype, op)."""
    coll = rng.choice(["allreduce", "allreduce", "reduce_scatter", "all_gather"])
    P = int(rng.choice([2, 3, 4, 5, 6, 7, 8, 9, 12, 16]))
    L = nu.ceil_log2(P)
    pow2 = P & (P - 1) == 0
    algos = ["direct", "ring", "generalized"] + (["rh_rd", "generalized_xor"] if pow2 else [])
    if coll == "allreduce":
        algos += ["rh_rd", "rd", "binomial", "ahc", "chain"]
    algo = str(rng.choice(sorted(set(algos))))
    knob, steps, factors, groups = 0, 0, None, None
    if algo == "generalized":
        steps = int(rng.choice([0, 0, rng.integers(L, max(L, P - 1) + 1)]))
        fs = factorizations(P)
        factors = fs[int(rng.integers(len(fs)))]
        if coll == "allreduce":
            knob = int(rng.integers(0, (steps or L) + 1))
    elif algo == "generalized_xor" and coll == "allreduce":
        knob = int(rng.integers(0, L + 1))
    elif algo == "chain":
        knob = int(rng.integers(1, 12))
    elif algo == "ahc":
        g = int(rng.integers(1, P)) if P > 2 else 1
        groups = [g, P - g] if P > 2 else [P]
    n = int(rng.choice([1, 3, P - 1, P + 1, 17, 64, 211]))
    batch = int(rng.choice([1, 1, 3]))
    dtype = str(rng.choice(["int32", "fp32", "bf16"]))
    ops = ["sum", "max"] + (["avg"] if dtype != "int32" else [])
    op = "sum" if coll == "all_gather" else str(rng.choice(ops))
    return coll, algo, knob, steps, factors, groups, P, n, batch, dtype, op


def oracle_result(coll, algo, knob, steps, factors, groups, P, n, batch, dtype, op, x):
    xb = x.reshape(P, batch, n)
    kw = {}
    if steps:
        kw["steps"] = steps
    if factors:
        kw["factors"] = tuple(factors)
    if coll == "reduce_scatter":
        return sch.reduce_scatter(xb, algo, dtype, op, **kw)
    if coll == "all_gather":
        return sch.all_gather(xb, algo, dtype, **kw).reshape(P, batch * n)
    return sch.allreduce(xb, algo, dtype, op, knob=knob, groups=groups, **kw).reshape(P, batch * n)


def as_bits(a):
    a = np.asarray(a)
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)


@pytest.mark.parametrize("seed", range(8))
def test_random_cases_match_oracle(seed):
    rng = np.random.default_rng(1000 + seed)
    for _ in range(25):
        coll, algo, knob, steps, factors, groups, P, n, batch, dtype, op = draw(rng)
        x = inputs.make(dtype, P, n * batch, seed=int(rng.integers(1 << 30)))
        want = oracle_result(coll, algo, knob, steps, factors, groups, P, n, batch, dtype, op, x)
        s = A.ar_schedule_build(A.make_call(P, n, dtype, op, algo, knob, "literal", batch=batch,
                                            groups=groups if algo == "ahc" else factors, collective=coll, steps=steps))
        interp_op = "sum" if coll == "all_gather" else op
        outs = [run_table(x, s.export(), dtype, interp_op, n, batch=batch)]
        if s.info().fused_ok:
            outs.append(run_fused(x, *s.fused_export(), dtype, interp_op, n, batch=batch))
        case = (coll, algo, knob, steps, factors, groups, P, n, batch, dtype, op)
        for got in outs:
            if coll == "reduce_scatter":
                own = np.arange(n) // (-(-n // P))
                got = got.reshape(P, batch, n)[own, :, np.arange(n)].T
            assert np.array_equal(as_bits(got), as_bits(want)), case
