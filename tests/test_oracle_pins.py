"""Pins for the CPU oracle: facts the pages and the mathematics fix.

None of these re-types the oracle's own formula; each checks it against
something independent: brute force, counts printed in the pages' prose, hand
derivations stored under tests/golden/, structural equivalences between
schedules that the oracle implements separately, closed error bounds, or an
independent bf16 rounding. A few tests plant a plausible mistake in the
oracle (monkeypatched, on the CPU) and check that the pins catch it.
"""
import math

import numpy as np
import pytest

import oracle
from oracle import cost, numerics as nu, schedules as sch
from oracle.net import partition
from synth import inputs

ALGOS_ANY_P = ("direct", "ring", "rh_rd", "rd", "binomial", "generalized", "ahc")


def knobs(algo, P):
    return range(nu.ceil_log2(P) + 1) if algo.startswith("generalized") else [0]


def default_groups(P):
    return [P] if P < 3 else [P // 3 + 1, P - (P // 3 + 1)]


def run(x, algo, dtype, op, r=0, P=None, groups=None, **kw):
    P = x.shape[0]
    if algo == "ahc" and groups is None:
        groups = default_groups(P)
    return oracle.allreduce(x, algo, dtype, op, knob=r, groups=groups, **kw)


# --------------------------------------------------------------------------
# exact results: int32 sum / max in every dtype equal brute force, all ranks
# --------------------------------------------------------------------------
@pytest.mark.parametrize("algo", ALGOS_ANY_P + ("generalized_xor",))
@pytest.mark.parametrize("P", [1, 2, 3, 4, 5, 6, 7, 8, 9, 12, 13, 16])
def test_exact_results_equal_brute_force(algo, P):
    if algo == "generalized_xor" and P & (P - 1):
        pytest.skip("XOR group needs a power of two")
    for n in (1, 5, 37, 100):
        for r in knobs(algo, P):
            xi = inputs.make("int32", P, n, seed=1000 * P + n)
            for op in ("sum", "max"):
                y = run(xi, algo, "int32", op, r)
                assert np.array_equal(y, np.broadcast_to(nu.brute_force(xi, "int32", op), y.shape))
            for dt in ("fp32", "bf16"):
                xf = inputs.make(dt, P, n, seed=7 * P + n)
                y = run(xf, algo, dt, "max", r)
                bf = nu.brute_force(xf, dt, "max")
                assert np.array_equal(y.view(np.uint32 if dt == "fp32" else np.uint16),
                                      np.broadcast_to(bf, y.shape).view(np.uint32 if dt == "fp32" else np.uint16))


def test_int32_wraps_modulo_2_32():
    x = np.array([[2**31 - 1, -(2**31)], [1, -1], [5, 0]], dtype=np.int32)
    for algo in ("ring", "rd", "binomial", "direct", "generalized"):
        y = run(x, algo, "int32", "sum")
        assert y[:, 0].tolist() == [-(2**31) + 5] * 3
        assert y[:, 1].tolist() == [2**31 - 1] * 3


def test_max_prefers_positive_zero():
    x = np.zeros((5, 4), dtype=np.float32)
    x[0] = -0.0
    x[3] = -0.0
    for algo in ALGOS_ANY_P:
        y = run(x, algo, "fp32", "max")
        assert not np.signbit(y).any(), algo
    allneg = np.full((4, 3), -0.0, dtype=np.float32)
    assert np.signbit(run(allneg, "ring", "fp32", "max")).all()


def test_empty_and_single_rank():
    for algo in ALGOS_ANY_P:
        x = inputs.make("fp32", 4, 0)
        assert run(x, algo, "fp32", "sum").shape == (4, 0)
        x1 = inputs.make("fp32", 1, 9)
        assert np.array_equal(run(x1, algo, "fp32", "sum"), x1)


# --------------------------------------------------------------------------
# floating-point sums: closed error bound, exact on integer-valued data
# --------------------------------------------------------------------------
@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
@pytest.mark.parametrize("algo", ALGOS_ANY_P)
def test_fp_sum_within_closed_bound(algo, dtype):
    for P in (3, 7, 8, 13):
        n = 257
        x = inputs.make(dtype, P, n, seed=P)
        ref = nu.fp64_reference(x, dtype)
        bound = nu.sum_error_bound(x, dtype)
        for r in knobs(algo, P):
            y = run(x, algo, dtype, "sum", r)
            yf = nu.bf16_to_f32(y) if dtype == "bf16" else y
            assert np.all(np.abs(yf.astype(np.float64) - ref[None]) <= bound[None] + 1e-300), (algo, P, r)


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_fp_sum_exact_when_no_rounding(dtype):
    # integers in [-8, 8]: every partial sum is exact in fp32 and the result is
    # exact in bf16 (|sum| <= 8 P < 256), so every schedule equals the true sum
    for algo in ALGOS_ANY_P:
        for P in (5, 8, 12):
            x = inputs.make(dtype, P, 64, seed=3, dist="small_int")
            for r in knobs(algo, P):
                y = run(x, algo, dtype, "sum", r)
                yf = nu.bf16_to_f32(y) if dtype == "bf16" else y
                truth = nu.fp64_reference(x, dtype)
                assert np.array_equal(yf.astype(np.float64), np.broadcast_to(truth, yf.shape))


def test_fp32_sum_depends_on_schedule():
    # the blog page's numerics section: summation order changes the last bits
    x = inputs.make("fp32", 7, 4096, seed=11)
    a = run(x, "ring", "fp32", "sum")
    b = run(x, "direct", "fp32", "sum")
    assert not np.array_equal(a, b)


# --------------------------------------------------------------------------
# step counts and traffic printed by the pages
# --------------------------------------------------------------------------
def _formula(expr, P, r=0):
    Pp = 1 << (P.bit_length() - 1)
    env = dict(P=P, L=nu.ceil_log2(P), Pp=Pp, r=r, fold=2 if P != Pp else 0,
               log2=lambda v: int(math.log2(v)))
    return eval(expr, {"__builtins__": {}}, env)


def test_step_counts_from_golden(golden):
    for algo, expr, *_ in golden("step_counts.txt"):
        for P in (2, 3, 5, 6, 7, 8, 12, 16, 24, 127):
            for r in knobs(algo, P):
                _, st = run(np.zeros((P, P), dtype=np.int32), algo, "int32", "sum", r, return_stats=True)
                assert st["steps"] == _formula(expr, P, r), (algo, P, r)


def test_config_step_counts():
    # 5-rank ring: 8 steps; 8-rank halving/doubling: 6; 7-rank generalized: 6..3;
    # 3/6/12/24-rank doubling with fold: 3/4/5/6, binomial: 4/6/8/10
    z = lambda P: np.zeros((P, 4), dtype=np.int32)  # noqa: E731
    assert run(z(5), "ring", "int32", "sum", return_stats=True)[1]["steps"] == 8
    assert run(z(8), "rh_rd", "int32", "sum", return_stats=True)[1]["steps"] == 6
    assert [run(z(7), "generalized", "int32", "sum", r, return_stats=True)[1]["steps"] for r in range(4)] == [6, 5, 4, 3]
    assert [run(z(P), "rd", "int32", "sum", return_stats=True)[1]["steps"] for P in (3, 6, 12, 24)] == [3, 4, 5, 6]
    assert [run(z(P), "binomial", "int32", "sum", return_stats=True)[1]["steps"] for P in (3, 6, 12, 24)] == [4, 6, 8, 10]
    st = run(np.zeros((192, 256), dtype=np.int32), "ahc", "int32", "sum", groups=[64, 128], return_stats=True)[1]
    assert st["steps"] == 2 * 127 + 2


def test_ring_traffic_per_rank():
    # blog page, "The ring algorithm": each GPU sends 2(N-1)S/N and receives the same
    for P, n in ((4, 4096), (8, 1 << 12), (7, 7 * 33)):
        _, st = run(np.zeros((P, n), dtype=np.int32), "ring", "int32", "sum", return_stats=True)
        assert (st["sent"].sum(0) == 2 * (P - 1) * n // P).all()
        assert (st["recv"].sum(0) == 2 * (P - 1) * n // P).all()
    # ragged 5-rank, 4096-element case: 6552 or 6556 per rank, 2(P-1)n in total
    _, st = run(np.zeros((5, 4096), dtype=np.int32), "ring", "int32", "sum", return_stats=True)
    per = st["sent"].sum(0)
    assert set(per.tolist()) == {6552, 6556} and per.sum() == 2 * 4 * 4096


def test_direct_root_carries_everything():
    # blog page, naive approach: the root receives (N-1)S and sends (N-1)S
    P, n = 6, 100
    _, st = run(np.zeros((P, n), dtype=np.int32), "direct", "int32", "sum", return_stats=True)
    assert st["recv"].sum(0)[0] == (P - 1) * n and st["sent"].sum(0)[0] == (P - 1) * n
    assert (st["sent"].sum(0)[1:] == n).all()


@pytest.mark.parametrize("algo", ["direct", "ring", "rh_rd", "rd", "binomial"])
def test_single_port(algo):
    # generalized-Allreduce paper, cost model: full-duplex peer-to-peer links,
    # one communication at a time per process
    for P in (3, 5, 8, 12):
        _, st = run(np.zeros((P, 3 * P), dtype=np.int32), algo, "int32", "sum", return_stats=True)
        for pairs in st["peers"]:
            srcs = [s for s, _ in pairs]
            dsts = [d for _, d in pairs]
            assert len(srcs) == len(set(srcs)) and len(dsts) == len(set(dsts))


def test_generalized_single_port_and_shift():
    for P in (5, 7, 12):
        for r in knobs("generalized", P):
            _, st = run(np.zeros((P, P), dtype=np.int32), "generalized", "int32", "sum", r, return_stats=True)
            assert st["steps"] == 2 * nu.ceil_log2(P) - r


def test_generalized_r0_moves_what_the_ring_moves():
    # paper, bandwidth-optimal section: transmitted data and calculations stay
    # the same as for the ring: (P-1) parts sent per phase, (P-1) parts combined
    for P in (3, 5, 6, 7, 9, 12, 127):
        _, st = run(np.zeros((P, P), dtype=np.int32), "generalized", "int32", "sum", 0, return_stats=True)
        assert sum(st["reduction_sent_parts"]) == P - 1
        assert sum(st["reduction_reduced_parts"]) == P - 1
        assert sum(st["distribution_sent_parts"]) == P - 1


def test_generalized_r1_increments():
    # paper, intermediate-steps section: one more result vector adds u to the
    # data sent on each reduction step, and 2u of calculations on steps where
    # N_i is even, u where it is odd. Readings: on the last step (N = 2) only
    # one new combination exists, so +u (the paper's worst case then totals
    # (2L - 2) u). For even P the shifted schedule coincides with the base one
    # until the first odd N_i leaves a vector out, so those early even steps add
    # only u; the prose rule is checked exactly for odd P.
    for P in (5, 6, 7, 11, 12, 13, 127):
        L, N, h = sch._levels(P)
        _, s0 = run(np.zeros((P, P), dtype=np.int32), "generalized", "int32", "sum", 0, return_stats=True)
        _, s1 = run(np.zeros((P, P), dtype=np.int32), "generalized", "int32", "sum", 1, return_stats=True)
        ds = np.subtract(s1["reduction_sent_parts"], s0["reduction_sent_parts"])
        dr = np.subtract(s1["reduction_reduced_parts"], s0["reduction_reduced_parts"])
        assert (ds == 1).all(), (P, ds)
        assert dr.sum() <= 2 * L - 2
        if P % 2:
            for i in range(L):
                want = 1 if (N[i] % 2 or i == L - 1) else 2
                assert dr[i] == want, (P, i, dr)


def test_generalized_extra_send_formula():
    # paper, intermediate-steps section: extra data (2^r - 1) ceil(log P) u;
    # extra calculations at most (2^r - 1)(2 ceil(log P) - 2) u
    for P, rmax in ((7, 2), (127, 6)):
        L = nu.ceil_log2(P)
        for r in range(rmax + 1):
            _, st = run(np.zeros((P, P), dtype=np.int32), "generalized", "int32", "sum", r, return_stats=True)
            assert sum(st["reduction_sent_parts"]) - (P - 1) == (2**r - 1) * L
            assert sum(st["reduction_reduced_parts"]) - (P - 1) <= (2**r - 1) * (2 * L - 2)


def test_latency_optimal_sends_everything_each_step():
    # paper, latency-optimal section: on each step all data vectors are sent
    for P in (5, 7, 8, 12):
        L = nu.ceil_log2(P)
        _, st = run(np.zeros((P, P), dtype=np.int32), "generalized", "int32", "sum", L, return_stats=True)
        assert st["reduction_sent_parts"] == [P] * L
        assert st["distribution_sent_parts"] == []


# --------------------------------------------------------------------------
# structure: trees, equivalences, AHC layout
# --------------------------------------------------------------------------
def trees(algo, P, r=0, n=None, **kw):
    n = P if n is None else n
    y, st = run(np.zeros((P, n), dtype=np.int32), algo, "int32", "sum", r, symbolic=True, return_stats=True, **kw)
    return y, st["algebra"]


def test_binomial_tree_from_golden(golden):
    want = golden("binomial_p6.txt")[0][0]
    y, alg = trees("binomial", 6, n=1)
    assert all(alg.show(y[p, 0]) == want for p in range(6))


def test_ring_part_chain_and_owner():
    # blog page ring: part k starts at rank k and gathers ranks k+1, k+2, ...;
    # rank r ends the reduce-scatter owning part (r + 1) mod N
    P = 6
    y, alg = trees("ring", P)
    for k in range(P):
        node = y[0, k]
        order = []
        while alg.children(node) is not None:
            a, b = alg.children(node)
            leaf, rest = (a, b) if alg.children(a) is None and alg.children(b) is not None else (b, a)
            if alg.children(a) is None and alg.children(b) is None:
                order += [max(a, b) if (min(a, b) - k) % P == 0 else min(a, b)]
                order += [k]
                break
            order.append(leaf)
            node = rest
        order = order[::-1]
        assert order == [(k + j) % P for j in range(P)], (k, order)


def test_rh_tree_pairs_half_distance_first():
    y, alg = trees("rh_rd", 8)
    assert alg.show(y[0, 0]) == "(((x0+x4)+(x2+x6))+((x1+x5)+(x3+x7)))"
    assert len({y[p, i] for p in range(8) for i in range(8)}) == 1


@pytest.mark.parametrize("dtype", ["fp32", "bf16"])
def test_xor_generalized_equals_halving_and_doubling(dtype):
    # paper: with the self-inverse group of Table 1.b the bandwidth-optimal
    # version is Recursive Halving and the latency-optimal one is Recursive
    # Doubling; two independently written replays must agree bit for bit
    for P in (2, 4, 8, 16):
        x = inputs.make(dtype, P, 3 * P + 5, seed=P)
        L = nu.ceil_log2(P)
        g0 = run(x, "generalized_xor", dtype, "sum", 0)
        gL = run(x, "generalized_xor", dtype, "sum", L)
        assert np.array_equal(g0, run(x, "rh_rd", dtype, "sum"))
        assert np.array_equal(gL, run(x, "rd", dtype, "sum"))
        assert np.array_equal(g0, gL)


def test_rd_fold_tree_matches_halving_fold():
    for P in (3, 5, 6, 12, 24):
        x = inputs.make("fp32", P, 40, seed=P)
        assert np.array_equal(run(x, "rd", "fp32", "sum"), run(x, "rh_rd", "fp32", "sum"))


def test_generalized_cyclic_rank_trees():
    # every rank's part is a complete balanced tree over all P ranks; for a power
    # of two the shifted trees coincide; otherwise r >= 1 gives different trees
    # at different ranks (the pages only say order changes bits)
    for P, want in ((6, [1, 2, 3, 3]), (7, [1, 2, 4, 7]), (8, [1, 1, 1, 1]), (16, [1] * 5)):
        got = []
        for r in range(nu.ceil_log2(P) + 1):
            y, alg = trees("generalized", P, r)
            for p in range(P):
                for i in range(P):
                    assert alg.leaves(y[p, i]) == list(range(P))
                    assert alg.depth(y[p, i]) == nu.ceil_log2(P)
            got.append(len({y[p, 0] for p in range(P)}))
        assert got == want


def test_generalized_r1_result_map_p7():
    # paper Fig. 6 idea: with two results t^0 q and t^1 q the first
    # distribution step is skipped; the remaining copies fan them out
    _, st = run(np.zeros((7, 7), dtype=np.int32), "generalized", "int32", "sum", 1, return_stats=True)
    assert st["J"] == [0, 1]
    assert st["src"] == [0, 1, 0, 1, 1, 0, 1]


def test_ahc_chunks_from_golden(golden):
    for gs, lcm, G, chunks in golden("ahc_chunks.txt"):
        groups = [int(v) for v in gs.split(",")]
        assert sch.ahc_chunks(groups) == int(chunks)
        assert math.lcm(*groups) == int(lcm) and len(groups) == int(G)
    assert sch.ahc_chunks([64, 128]) == 256


def test_ahc_pieces_from_golden(golden):
    want = [(int(a), int(b)) for a, b in golden("ahc_pieces_2_3.txt")]
    got = [(b0, b1) for b0, b1, _ in sch.ahc_pieces([2, 3])]
    assert got == want
    # every piece is a whole number of G chunks
    for b0, b1, _ in sch.ahc_pieces([64, 128]):
        assert (b1 - b0) % 2 == 0


def test_ahc_single_group_is_ring():
    x = inputs.make("fp32", 5, 103, seed=2)
    assert np.array_equal(run(x, "ahc", "fp32", "sum", groups=[5]), run(x, "ring", "fp32", "sum"))


def test_ahc_two_groups_tree():
    # groups (2, 3): every rank ends with ((chain of group A) + (chain of group B))
    y, alg = trees("ahc", 5, n=12, groups=[2, 3])
    for p in range(5):
        for e in range(12):
            a, b = alg.children(y[p, e])
            la, lb = alg.leaves(a), alg.leaves(b)
            assert sorted([la, lb]) == [[0, 1], [2, 3, 4]]


def test_partition_from_golden(golden):
    for length, N, sizes in golden("ring_split.txt"):
        got = [hi - lo for lo, hi in partition(int(length), int(N))]
        assert got == [int(v) for v in sizes.split(",")]


# --------------------------------------------------------------------------
# batching and sampling
# --------------------------------------------------------------------------
@pytest.mark.parametrize("algo", ["rd", "binomial", "direct"])
def test_batched_equals_long_vector(algo):
    # chunk-less schedules treat 10^4 x 106 as one long vector, bit for bit
    for P in (3, 6, 12):
        B, ln = 37, 106
        x = inputs.make("fp32", P, B * ln, seed=P, dist="uniform_pm1")
        long = run(x, algo, "fp32", "sum")
        per = run(x.reshape(P, B, ln), algo, "fp32", "sum", n=ln)
        assert np.array_equal(per.reshape(P, B * ln), long)


@pytest.mark.parametrize("algo", ALGOS_ANY_P + ("generalized_xor",))
def test_sampled_equals_full(algo):
    P = 8
    n = 1001
    x = inputs.make("fp32", P, n, seed=5)
    idx = inputs.sample_indices(n, P, count=50, seed=2)
    for r in knobs(algo, P):
        full = run(x, algo, "fp32", "sum", r)
        part = run(x[:, idx], algo, "fp32", "sum", r, n=n, idx=idx)
        assert np.array_equal(full[:, idx], part)


# --------------------------------------------------------------------------
# bf16 conversions, against an independent rounding and printed bit patterns
# --------------------------------------------------------------------------
def test_bf16_widening_known_patterns():
    pats = np.array([0x3F80, 0xC000, 0x3F81, 0x0001, 0x7F7F, 0x8000], dtype=np.uint16)
    want = [1.0, -2.0, 1.0 + 2.0**-7, 2.0**-133, (2 - 2.0**-7) * 2.0**127, -0.0]
    got = nu.bf16_to_f32(pats)
    assert [float(v) for v in got] == want
    assert np.signbit(got[-1])


def test_bf16_rounding_matches_frexp_rounding():
    rng = np.random.default_rng(0)
    v = (rng.standard_normal(200_000) * np.exp(rng.uniform(-30, 30, 200_000))).astype(np.float32)
    m, e = np.frexp(v.astype(np.float64))  # v = m 2^e, 0.5 <= |m| < 1, 8 significant bits kept
    ref = np.ldexp(np.round(m * 256.0) / 256.0, e)  # numpy rounds half to even
    got = nu.bf16_to_f32(nu.f32_to_bf16(v)).astype(np.float64)
    assert np.array_equal(got, ref)
    # the input generator's independent rounding agrees too
    assert np.array_equal(nu.f32_to_bf16(v), inputs.fp32_to_bf16_bits(v))


def test_bf16_rounding_edge_patterns():
    def r(bits):
        return int(nu.f32_to_bf16(np.array([bits], dtype=np.uint32).view(np.float32))[0])
    assert r(0x3F808000) == 0x3F80  # tie, even upper stays
    assert r(0x3F818000) == 0x3F82  # tie, odd upper rounds up
    assert r(0x3F808001) == 0x3F81  # above the tie
    assert r(0x3F7FFFFF) == 0x3F80  # carry into the exponent
    assert r(0x7F7FFFFF) == 0x7F80  # largest finite rounds to infinity


# --------------------------------------------------------------------------
# cost-model arithmetic
# --------------------------------------------------------------------------
def test_worked_example_from_golden(golden):
    for N, S, bb, secs, tol in golden("worked_example.txt"):
        t = cost.estimated_allreduce_seconds(float(S), int(N), float(bb))
        assert abs(t - float(secs)) <= float(tol)


def test_bus_bandwidth_and_ring_bytes():
    assert cost.busbw(100.0, 8) == pytest.approx(175.0)
    assert cost.ring_bytes_per_rank(8, 800.0) == pytest.approx(1400.0)
    # cost model closed forms: r = 0 is the bandwidth-optimal cost
    assert cost.intermediate_time(7, 7e3, 0, 1.0, 1e-3, 1e-4) == pytest.approx(
        cost.bandwidth_optimal_time(7, 7e3, 1.0, 1e-3, 1e-4))
    # latency dominated -> fewest steps; bandwidth dominated -> r = 0
    assert cost.optimal_r(127, 425, 1e-5, 1e-10, 1e-12) == 6
    assert cost.optimal_r(127, 1e9, 1e-5, 1e-9, 1e-12) == 0


# --------------------------------------------------------------------------
# planted mistakes: the pins above must catch them
# --------------------------------------------------------------------------
def test_planted_floor_levels_is_caught(monkeypatch):
    def bad_levels(P, steps=None):
        L = nu.ceil_log2(P)
        N = [P]
        for _ in range(L):
            N.append(max(N[-1] // 2, 1))  # floor instead of ceil
        return L, N, [N[i] // 2 for i in range(L)]
    monkeypatch.setattr(sch, "_levels", bad_levels)
    x = inputs.make("int32", 7, 21, seed=1)
    try:
        y = run(x, "generalized", "int32", "sum", 0)
    except (KeyError, IndexError):
        return  # the broken level sequence cannot even place every result
    assert not np.array_equal(y, np.broadcast_to(nu.brute_force(x, "int32", "sum"), y.shape))


def test_planted_ring_direction_is_caught(monkeypatch):
    orig = sch._ring

    def bad_ring(net):
        # the reduce lap runs against the ring direction (part k hops k -> k - 1)
        # while the gather lap still starts from rank k - 1 and runs with it
        P, n = net.P, net.n
        parts = partition(n, P)
        for t in range(P - 1):
            net.step([((k - t) % P, (k - t - 1) % P, *parts[k], oracle.net.REDUCE) for k in range(P)])
        for t in range(P - 1):
            net.step([((k - 1 + t) % P, (k + t) % P, *parts[k], oracle.net.COPY) for k in range(P)])
    monkeypatch.setattr(sch, "_ring", bad_ring)
    x = inputs.make("int32", 5, 20, seed=1)
    y = run(x, "ring", "int32", "sum")
    assert not np.array_equal(y, np.broadcast_to(nu.brute_force(x, "int32", "sum"), y.shape))
    monkeypatch.setattr(sch, "_ring", orig)


def test_planted_rh_distance_order_is_caught(monkeypatch):
    # halving with distance 1 first is still a correct Allreduce but a different
    # tree; the equivalence with the XOR-group generalized algorithm catches it
    def bad(net):
        n, Pp = net.n, net.P
        L = Pp.bit_length() - 1
        parts = partition(n, Pp)

        def window(p, s):  # parts agreeing with p on the s lowest bits
            mask = (1 << s) - 1
            return [i for i in range(Pp) if (i & mask) == (p & mask)]
        for s in range(L):
            d = 1 << s
            net.step([(p, p ^ d, *parts[i], oracle.net.REDUCE)
                      for p in range(Pp) for i in window(p, s) if (i & d) != (p & d)])
        for s in reversed(range(L)):
            d = 1 << s
            net.step([(p, p ^ d, *parts[i], oracle.net.COPY) for p in range(Pp) for i in window(p, s + 1)])
    monkeypatch.setattr(sch, "_rh_rd", bad)
    x = inputs.make("fp32", 8, 64, seed=3)
    y = run(x, "rh_rd", "fp32", "sum")
    assert np.array_equal(y[0], y[0])
    xi = inputs.make("int32", 8, 64, seed=3)
    assert np.array_equal(run(xi, "rh_rd", "int32", "sum")[0], nu.brute_force(xi, "int32", "sum"))
    assert not np.array_equal(y, run(x, "generalized_xor", "fp32", "sum", 0))
