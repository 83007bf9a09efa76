"""Step-by-step replays of every Allreduce schedule on the pages (oracle).

Each replay drives the rank simulator of ``net`` (or, for the generalized
algorithm, the paper's own vector-and-placement formalism) through the
schedule's steps in the pages' order, then returns every rank's final buffer.
The per-element combination order therefore is exactly the schedule's.

Where a page leaves a step open, the reading taken is stated at the function.

Public entry point: ``allreduce(x, algo, dtype, op, ...)``.
"""
from __future__ import annotations

import math
from functools import reduce as _fold

import numpy as np

from .net import COPY, REDUCE, Net, partition
from .numerics import Algebra, Symbolic, ceil_log2

ALGOS = ("direct", "ring", "rh_rd", "rd", "binomial", "generalized", "generalized_xor", "ahc", "chain")


def _pow2_floor(P: int) -> int:
    return 1 << (P.bit_length() - 1)


# --------------------------------------------------------------------------
# direct: gather to one root, combine, broadcast
# --------------------------------------------------------------------------
def _direct(net: Net):
    """The naive one-root schedule of the all-reduce blog page ("A cost model for
    collectives": gather at GPU 0, sum, broadcast back).

    Reading: the page fixes no order for the root's combinations; the root
    folds the other ranks in rank order, x0 + x1, then + x2, ..., one incoming
    buffer per step (a rank receives one message per step), then sends the
    result to each rank in rank order.
    """
    P, n = net.P, net.n
    for s in range(1, P):
        net.step([(s, 0, 0, n, REDUCE)])
    for s in range(1, P):
        net.step([(0, s, 0, n, COPY)])


# --------------------------------------------------------------------------
# ring reduce-scatter + all-gather
# --------------------------------------------------------------------------
def _ring(net: Net):
    """Ring Allreduce ("The ring algorithm", all-reduce blog page; also the cyclic
    case of the straightforward algorithm, generalized-Allreduce paper,
    eqs. (14)-(16) and Fig. 5).

    The data is cut into P parts (ceil split) and every part makes two laps of
    the ring, one hop r -> r + 1 per step for all parts at once. Reduce lap:
    part k sets out from rank k; each rank it reaches adds its own copy of the
    part, so after P - 1 hops it rests at rank k - 1 holding every rank's
    contribution (that rank owns part k). Gather lap: the finished part k
    leaves its owner and hops on, each rank it reaches overwriting its copy,
    until after P - 1 more hops every rank has it.
    """
    P, n = net.P, net.n
    parts = partition(n, P)

    def lap(first_holder, kind):
        for t in range(P - 1):
            msgs = []
            for k in range(P):
                at = (first_holder(k) + t) % P  # where part k is before this hop
                msgs.append((at, (at + 1) % P, *parts[k], kind))
            net.step(msgs)

    lap(lambda k: k, REDUCE)            # part k starts at its first contributor, rank k
    lap(lambda k: (k - 1) % P, COPY)    # and leaves its owner, rank k - 1


# --------------------------------------------------------------------------
# fold-in for non-power-of-two P
# --------------------------------------------------------------------------
def _fold_in(net: Net) -> int:
    """Preparation step for P that is not a power of two (generalized-Allreduce
    paper, related-work paragraph on non-power-of-two process counts): the
    excess ranks hand their whole buffer to ranks that take part in the
    power-of-two algorithm.

    Reading: excess rank P' + j sends to rank j (j < P - P'), which adds it in.
    Returns P' (the largest power of two <= P).
    """
    P, n = net.P, net.n
    Pp = _pow2_floor(P)
    if P > Pp:
        net.step([(Pp + j, j, 0, n, REDUCE) for j in range(P - Pp)])
    return Pp


def _fold_out(net: Net, Pp: int):
    """Finalization step: rank j returns the result to excess rank P' + j."""
    P, n = net.P, net.n
    if P > Pp:
        net.step([(j, Pp + j, 0, n, COPY) for j in range(P - Pp)])


# --------------------------------------------------------------------------
# recursive halving reduce-scatter + recursive doubling all-gather
# --------------------------------------------------------------------------
def _rh_rd(net: Net):
    """Recursive Halving (bandwidth-optimal, 2 log P steps; generalized-Allreduce
    paper, introduction; it is the bandwidth-optimal generalized algorithm over
    the self-inverse group of Table 1.b).

    P' parts. Reduction step s = 0..L-1 with distance d = P' / 2^(s+1): rank p
    works on a window of 2d parts (those whose index agrees with p on all bits
    of value >= 2d); it sends the half whose bit d differs from p's to partner
    p XOR d and adds the partner's copy of the half it keeps. After L steps
    rank p holds the sum of part p. All-gather: the same distances in reverse
    order (d = 1, 2, ...), each rank copying its whole current window to
    p XOR d.

    Reading: the distance order (P'/2 first) is the one the generalized
    algorithm produces over the XOR group; the pages do not fix it otherwise.
    """
    Pp = _fold_in(net)
    _halving(net, Pp)
    _doubling(net, Pp)
    _fold_out(net, Pp)


def _halving(net: Net, Pp: int):
    """The reduction half of recursive halving over ranks 0..P'-1: afterwards
    rank p holds the complete part p of P' parts."""
    parts = partition(net.n, Pp)
    L = Pp.bit_length() - 1

    def rng(first_part: int, count: int):
        return parts[first_part][0], parts[first_part + count - 1][1]

    for s in range(L):
        d = Pp >> (s + 1)
        msgs = []
        for p in range(Pp):
            base = p & ~(2 * d - 1)
            give = base + (d if (p & d) == 0 else 0)  # half the partner keeps
            msgs.append((p, p ^ d, *rng(give, d), REDUCE))
        net.step(msgs)


def _doubling(net: Net, Pp: int):
    """The all-gather half: distances 1, 2, ..., each rank copying its whole
    current window of parts to p XOR d."""
    parts = partition(net.n, Pp)
    L = Pp.bit_length() - 1
    for s in reversed(range(L)):
        d = Pp >> (s + 1)
        msgs = []
        for p in range(Pp):
            base = p & ~(d - 1)
            msgs.append((p, p ^ d, parts[base][0], parts[base + d - 1][1], COPY))
        net.step(msgs)


# --------------------------------------------------------------------------
# recursive doubling
# --------------------------------------------------------------------------
def _rd(net: Net):
    """Recursive Doubling (latency-optimal, log P steps; generalized-Allreduce
    paper, introduction and the latency-optimal section, which identifies it
    with the latency-optimal generalized algorithm over Table 1.b's group).

    In step s (distance d = P' / 2^(s+1)) ranks p and p XOR d exchange their
    whole buffers and both combine. Non-power-of-two P uses the fold-in.
    Reading: distance order P'/2 first, as for recursive halving.
    """
    n = net.n
    Pp = _fold_in(net)
    L = Pp.bit_length() - 1
    for s in range(L):
        d = Pp >> (s + 1)
        net.step([(p ^ d, p, 0, n, REDUCE) for p in range(Pp)])
    _fold_out(net, Pp)


# --------------------------------------------------------------------------
# binomial tree reduce + broadcast
# --------------------------------------------------------------------------
def _binomial(net: Net):
    """Binomial-tree reduce ("Reduction Operator" page, the PRAM algorithm and its
    distributed-memory form) followed by a broadcast from rank 0.

    For k = 0..ceil(log2 P)-1, every still-active rank i whose bit k is set
    sends its value to i - 2^k and becomes inactive; an active rank with bit k
    clear and i + 2^k < P combines x_i <- x_i (+) x_{i+2^k}.

    Reading: the broadcast is the reverse of the reduce (the page says the
    same steps run backwards serve as a broadcast): for k from the top down,
    every rank i that is a multiple of 2^(k+1) with i + 2^k < P copies its
    buffer to i + 2^k.
    """
    P, n = net.P, net.n
    K = ceil_log2(P)
    active = [True] * P
    for k in range(K):
        b = 1 << k
        msgs = []
        for i in range(P):
            if not active[i]:
                continue
            if i & b:
                active[i] = False
            elif i + b < P:
                msgs.append((i + b, i, 0, n, REDUCE))
        net.step(msgs)
    for k in reversed(range(K)):
        b = 1 << k
        net.step([(i, i + b, 0, n, COPY) for i in range(0, P, 2 * b) if i + b < P])


# --------------------------------------------------------------------------
# pipelined chain reduce + pipelined chain broadcast
# --------------------------------------------------------------------------
def _chain(net: Net, m: int):
    """Pipelined reduction along a chain ("Reduction Operator" page, pipelined
    algorithm): the vector is cut into m pieces; unit i passes each piece to
    i - 1 one step after it arrived, combined with its own, so the root 0 holds
    the first piece after p - 1 steps and the last after p + m - 2. The
    Allreduce adds a broadcast from the root (same page, where the reduce result
    is distributed afterwards), pipelined the same way down the chain.

    Reading: in step t unit i sends piece t - (p - 1 - i) to i - 1; the
    broadcast starts after the reduce (no overlap), unit i forwarding piece
    t - i to i + 1 in its step t. Pieces follow the ceil split.
    """
    P, n = net.P, net.n
    pieces = partition(n, m)
    for t in range(P + m - 2):
        msgs = []
        for i in range(1, P):
            k = t - (P - 1 - i)
            if 0 <= k < m:
                msgs.append((i, i - 1, *pieces[k], REDUCE))
        net.step(msgs)
    for t in range(P + m - 2):
        msgs = []
        for i in range(P - 1):
            k = t - i
            if 0 <= k < m:
                msgs.append((i, i + 1, *pieces[k], COPY))
        net.step(msgs)


# --------------------------------------------------------------------------
# AHC: asymmetric hierarchical Allreduce
# --------------------------------------------------------------------------
def _ahc(net: Net, groups):
    """AHC (HCCL "AHC" page, Description, steps 1-3).

    Groups are contiguous rank ranges (neighbouring devices form a group). With G groups and Lc
    the least common multiple of the group sizes, the buffer is cut into
    Lc * G chunks (ceil split). Group a of size g sees the buffer as g
    segments of C / g chunks each.

    1. Ring reduce-scatter inside every group in parallel, segments as parts
       (the ring's rule: local rank l passes segment (l - t) mod g to l + 1).
       Segment k's partial sum ends at local rank (k - 1) mod g.
    2. The union of all groups' segment boundaries cuts the buffer into pieces;
       each piece lies in one segment of every group, and that segment's owner
       in each group are the page's logical devices that share an ID. They run an
       Allreduce per piece.
       Reading: the sub-algorithm is the ring (one of the three the page names;
       the other two are not described), over the owners in group order, with
       the piece split into G equal sub-pieces (every piece is a whole multiple
       of G chunks).
    3. Ring all-gather inside every group.
    Groups smaller than the largest finish their ring phases early and idle.
    """
    P, n = net.P, net.n
    G = len(groups)
    if sum(groups) != P or min(groups) < 1:
        raise ValueError("group sizes must be positive and sum to P")
    Lc = _fold(lambda a, b: a * b // math.gcd(a, b), groups)
    C = Lc * G
    chunks = partition(n, C)
    offs = [sum(groups[:a]) for a in range(G)]
    span = [C // g for g in groups]  # chunks per segment

    def erange(c0: int, c1: int):
        return chunks[c0][0], chunks[c1 - 1][1]

    def seg(a: int, k: int):
        return erange(k * span[a], (k + 1) * span[a])

    gmax = max(groups)
    for t in range(gmax - 1):
        msgs = []
        for a, g in enumerate(groups):
            if t < g - 1:
                for l in range(g):
                    msgs.append((offs[a] + l, offs[a] + (l + 1) % g, *seg(a, (l - t) % g), REDUCE))
        net.step(msgs)

    pieces = []
    for b0, b1, owners in ahc_pieces(groups):
        w = (b1 - b0) // G
        subs = [erange(b0 + s * w, b0 + (s + 1) * w) for s in range(G)]
        pieces.append(([offs[a] + owners[a] for a in range(G)], subs))
    for t in range(G - 1):
        net.step([(ow[s], ow[(s + 1) % G], *sub[(s - t) % G], REDUCE)
                  for ow, sub in pieces for s in range(G)])
    for t in range(G - 1):
        net.step([(ow[s], ow[(s + 1) % G], *sub[(s + 1 - t) % G], COPY)
                  for ow, sub in pieces for s in range(G)])

    for t in range(gmax - 1):
        msgs = []
        for a, g in enumerate(groups):
            if t < g - 1:
                for l in range(g):
                    msgs.append((offs[a] + l, offs[a] + (l + 1) % g, *seg(a, (l + 1 - t) % g), COPY))
        net.step(msgs)


def ahc_pieces(groups):
    """AHC phase-2 pieces as (first chunk, end chunk, owner local rank per group).

    The cut points are the union of every group's segment boundaries (the
    page's "segment ... along the data boundaries of individual NPUs"); in
    group a the piece lies in segment k_a, whose ring reduce-scatter partial
    ends at local rank (k_a - 1) mod g_a.
    """
    G = len(groups)
    Lc = _fold(lambda a, b: a * b // math.gcd(a, b), groups)
    C = Lc * G
    span = [C // g for g in groups]
    bounds = sorted({k * span[a] for a, g in enumerate(groups) for k in range(g + 1)})
    return [(b0, b1, [(b0 // span[a] - 1) % g for a, g in enumerate(groups)])
            for b0, b1 in zip(bounds[:-1], bounds[1:])]


def ahc_chunks(groups) -> int:
    """Number of chunks AHC cuts the buffer into: LCM of group sizes times G."""
    Lc = _fold(lambda a, b: a * b // math.gcd(a, b), groups)
    return Lc * len(groups)


# --------------------------------------------------------------------------
# generalized Allreduce over a transitive abelian group of order P
# --------------------------------------------------------------------------
def _levels(P: int, steps: int | None = None):
    """Vector counts of the base reduction: step i moves v_k, k in [N_i - h_i, N_i),
    onto v_{k - h_i}, and N_{i+1} = N_i - h_i. Returns (S, N, h) for S steps.

    S = ceil(log2 P) (default): the paper's halving, N_{i+1} = ceil(N_i / 2),
    h_i = floor(N_i / 2).

    S > ceil(log2 P): the paper's conclusion names a version with more than
    2 ceil(log P) steps and smaller pieces per step, up to the ring's 2(P - 1),
    without defining it. Reading: the same base step with smaller h_i. Any
    1 <= h_i <= floor(N_i / 2) keeps every target v_{k - h_i} below N_i - h_i
    and distinct. h_i spreads the P - 1 parts as evenly as the remaining steps
    allow: h_i = max(ceil((N_i - 1) / (S - i)), N_i - 2^(S - i - 1)). The
    second term is the least h that still lets the rest halve down to one
    vector. S = P - 1 gives h_i = 1: a ring-shaped chain.
    """
    L = ceil_log2(P)
    S = L if steps is None else steps
    if not L <= S <= max(P - 1, L):
        raise ValueError(f"steps must be in [{L}, {max(P - 1, L)}]")
    N, h = [P], []
    for i in range(S):
        if S == L:
            hi = N[i] // 2
        else:
            left = S - i
            hi = max(-(-(N[i] - 1) // left), N[i] - (1 << (left - 1)))
        if not 1 <= hi <= N[i] // 2:
            raise AssertionError("level sequence out of range")
        h.append(hi)
        N.append(N[i] - hi)
    return S, N, h


def _product_group(factors, P: int):
    """The abelian group Z_m1 x ... x Z_mt as a group T_P (generalized paper:
    any suitable group may replace the cyclic one, Table 1 and the
    bandwidth-optimal section). Element k is the mixed-radix number with digits
    (k mod m1, (k // m1) mod m2, ...); the operation adds digits modulo their
    radix. Returns vectorized (add, sub)."""
    f = tuple(int(m) for m in factors)
    if not f or any(m < 2 for m in f) or math.prod(f) != P:
        raise ValueError("group factors must be >= 2 with product P")

    def digits(x):
        x = np.asarray(x, dtype=np.int64)
        out = []
        for m in f:
            out.append(x % m)
            x = x // m
        return out

    def number(ds):
        x, w = 0, 1
        for d, m in zip(ds, f):
            x = x + (d % m) * w
            w *= m
        return x

    def add(a, b):
        return number([u + v for u, v in zip(digits(a), digits(b))])

    def sub(a, b):
        return number([u - v for u, v in zip(digits(a), digits(b))])
    return add, sub


def _generalized(alg, xacc: np.ndarray, n: int, idx: np.ndarray, r: int, group, phase: str = "all",
                 steps: int | None = None):
    """Generalized Allreduce (generalized-Allreduce paper: bandwidth-optimal
    section eqs. (17)-(25), intermediate steps eqs. (26)-(36) and Fig. 6,
    latency-optimal section eqs. (38)-(44)). The equations are missing from the
    extracted text; this is the reading reconstructed from its prose.

    Placements. The group element t_j sends rank q to q + j (cyclic group,
    generator q -> q + 1 as in Fig. 2) or to q XOR j (the self-inverse group
    of Table 1.b, P a power of two). A distributed vector at placement j holds
    part i at rank t_j(i). The initial data matrix splits into P such vectors
    d_j (part i of rank t_j(i)'s buffer).

    Base reduction S_0 over vectors v_0..v_{N-1} (v_k = d_k initially): in step
    i, for k in [N_i - h_i, N_i), v_k is moved onto v_{k - h_i}'s placement
    (every rank sends its part of v_k to one rank, q - h_i) and combined into
    it. When N_i is odd, v_0 sits the step out (the paper names the first vector).
    After L = ceil(log2 P) steps v_0 is the sum at placement 0: rank i holds
    part i (a reduce-scatter).

    Knob r (removed distribution steps): the schedules S_j for j in
    J_r = {0 .. N_{L-r} - 1} run together; S_j is S_0 with every vector's
    placement shifted by j and the same communication operators. Reading: J_r
    is the smallest result set that lets the distribution skip r steps; it
    has 2^r members when N_{L-r} = 2^r. Identical vectors (same placement, same
    combination tree) are sent and combined once; distinct vectors on one
    placement are kept apart (the paper's q* and q').

    Distribution: the reduction steps L-r-1 .. 0 reversed, copying instead of
    combining: v_k <- v_{k - h_i} moved back (rank q sends to q + h_i).
    Steps: 2L - r. r = L is the latency-optimal version (no distribution).

    phase "reduce" runs only the reduction with r = 0 (the reduce-scatter the
    paper notes at its end); phase "gather" runs only the distribution with
    r = 0, starting from placement 0 = every rank's own part (an all-gather).

    Returns (per-rank outputs (P, B, m), stats dict with step counts and the
    per-step number of distinct parts sent / combined per rank).
    """
    P = xacc.shape[0]
    L, N, h = _levels(P, steps)  # L: reduction steps
    if not 0 <= r <= L:
        raise ValueError(f"knob r must be in [0, {L}]")
    if group == "cyclic":
        place = lambda k, j: (k + j) % P  # noqa: E731
        owner = lambda p, i: (p - i) % P  # placement held by rank p at part i  # noqa: E731
        ranks_of = lambda t: (t + np.arange(P)) % P  # rank holding part a of placement t  # noqa: E731
    elif group == "xor":
        if P & (P - 1):
            raise ValueError("the XOR group needs P to be a power of two")
        place = lambda k, j: k ^ j  # noqa: E731
        owner = lambda p, i: p ^ i  # noqa: E731
        ranks_of = lambda t: t ^ np.arange(P)  # noqa: E731
    else:
        add, sub = _product_group(group, P)
        place = add
        owner = sub
        ranks_of = lambda t: add(t, np.arange(P))  # noqa: E731

    c = -(-n // P) if n else 1
    part_of = (np.asarray(idx, dtype=np.int64) // c) if n else np.zeros(0, dtype=np.int64)
    cols = np.arange(len(idx))
    xt = np.transpose(xacc, (0, 2, 1))  # (P, m, B)

    def diag(j: int):
        # element at offset e (in part i) comes from rank t_j(i)
        return xt[place(part_of, j), cols].T if len(idx) else xacc[0, :, :0].copy()

    if phase not in ("all", "reduce", "gather"):
        raise ValueError(phase)
    if phase != "all" and r != 0:
        raise ValueError("the reduce-scatter and all-gather halves use r = 0")
    J = list(range(N[L - r]))
    sym = Symbolic(P)  # diagonal-level shadow, for dedupe and traffic counts
    sent_steps, red_steps = [], []
    # per-rank element counters: a vector at placement t is spread over all
    # ranks, part a on rank ranks_of(t)[a], so moving it moves every part once
    plen = np.array([hi - lo for lo, hi in partition(n, P)], dtype=np.int64)
    el_sent, el_recv, el_red = [], [], []
    vals = {j: [diag(place(k, j)) for k in range(P)] for j in J}
    syms = {j: [place(k, j) for k in range(P)] for j in J}
    built = set()  # (placement, tree) combined in an earlier step: not sent or combined again
    for i in range(L if phase != "gather" else 0):
        sends, reds, msgs = set(), set(), set()
        new_vals, new_syms = {}, {}
        for j in J:
            v, s = list(vals[j]), list(syms[j])
            for k in range(N[i] - h[i], N[i]):
                s[k - h[i]] = sym.node(syms[j][k - h[i]], syms[j][k])
                v[k - h[i]] = alg.op(vals[j][k - h[i]], vals[j][k])
                if (place(k - h[i], j), s[k - h[i]]) in built:
                    continue
                sends.add((place(k, j), syms[j][k]))
                msgs.add((place(k, j), syms[j][k], place(k - h[i], j)))
                reds.add((place(k - h[i], j), s[k - h[i]]))
            new_vals[j], new_syms[j] = v, s
        vals, syms = new_vals, new_syms
        built |= reds
        sent_steps.append(len(sends))
        red_steps.append(len(reds))
        es, er, ed = (np.zeros(P, dtype=np.int64) for _ in range(3))
        for t_from, _, t_to in msgs:
            es[ranks_of(t_from)] += plen
            er[ranks_of(t_to)] += plen
        for t_to, _ in reds:
            ed[ranks_of(t_to)] += plen
        el_sent.append(es)
        el_recv.append(er)
        el_red.append(ed)
    results = {j: vals[j][0] for j in J}  # result j sits at placement j

    src = {j: j for j in J}
    copy_steps = []
    if phase == "reduce":
        stats = dict(steps=L, sent=np.array(el_sent).reshape(-1, P), recv=np.array(el_recv).reshape(-1, P),
                     reduced=np.array(el_red).reshape(-1, P))
        return results[0], stats
    for i in reversed(range(L - r)):
        es, er = np.zeros(P, dtype=np.int64), np.zeros(P, dtype=np.int64)
        for k in range(N[i] - h[i], N[i]):
            src[k] = src[k - h[i]]
            es[ranks_of(k - h[i])] += plen
            er[ranks_of(k)] += plen
        copy_steps.append(h[i])
        el_sent.append(es)
        el_recv.append(er)
        el_red.append(np.zeros(P, dtype=np.int64))
    out = np.empty_like(xacc)
    src_of = np.array([src[k] for k in range(P)])
    for p in range(P):
        if len(idx):
            sel = src_of[owner(p, part_of)]
            for j in J:
                m = sel == j
                if m.any():
                    out[p][:, m] = results[j][:, m]
    stats = dict(
        steps=(L if phase != "gather" else 0) + (L - r),
        sent=np.array(el_sent).reshape(-1, P),
        recv=np.array(el_recv).reshape(-1, P),
        reduced=np.array(el_red).reshape(-1, P),
        reduction_sent_parts=sent_steps,
        reduction_reduced_parts=red_steps,
        distribution_sent_parts=copy_steps,
        J=J,
        src=[src[k] for k in range(P)],
    )
    return out, stats


# --------------------------------------------------------------------------
# entry point
# --------------------------------------------------------------------------
def allreduce(x: np.ndarray, algo: str, dtype: str, op: str = "sum", knob: int = 0,
              groups=None, n: int | None = None, idx=None, symbolic: bool = False,
              return_stats: bool = False, steps: int | None = None, factors=None):
    """Replay one Allreduce schedule on the CPU.

    x       (P, m) or (P, B, m): each rank's buffer (B independent instances of
            length n), restricted to the element offsets ``idx`` (default: all
            n offsets). int32 / fp32 arrays, bf16 as uint16 bit patterns.
    algo    one of ALGOS; ``knob`` is r for the generalized algorithm;
            ``groups`` the AHC group sizes (contiguous ranks); ``steps`` the
            generalized algorithm's reduction steps (default ceil(log2 P));
            ``factors`` (m1, ..., mt) its group Z_m1 x ... x Z_mt (default Z_P).
    symbolic  ignore the values and return, per rank and offset, the id of the
            combination tree (leaves = ranks) in ``stats['algebra']``.
    Returns the per-rank outputs in x's shape (and a stats dict if asked).
    """
    x = np.asarray(x)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[:, None, :]
    P, B, m = x.shape
    if n is None:
        n = m
    idx = np.arange(n, dtype=np.int64) if idx is None else np.asarray(idx, dtype=np.int64)
    if len(idx) != m:
        raise ValueError("idx must list one offset per sampled element")
    if symbolic:
        alg = Symbolic(P)
        xacc = np.empty((P, B, m), dtype=object)
        for p in range(P):
            xacc[p] = p
    else:
        alg = Algebra(dtype, op)
        xacc = np.stack([alg.load(x[p]) for p in range(P)])

    if P == 1 or n == 0:
        out, stats = xacc.copy(), dict(steps=0)
    elif algo in ("generalized", "generalized_xor"):
        if steps is not None and algo == "generalized_xor" and steps != ceil_log2(P):
            raise ValueError("more steps are defined for the cyclic group only")
        grp = "cyclic" if algo == "generalized" else "xor"
        if factors:
            if algo != "generalized":
                raise ValueError("group factors apply to the generalized algorithm")
            grp = tuple(factors)
        out, stats = _generalized(alg, xacc, n, idx, knob, grp, steps=steps)
    else:
        net = Net(alg, xacc.copy(), n, idx)
        if algo == "direct":
            _direct(net)
        elif algo == "ring":
            _ring(net)
        elif algo == "rh_rd":
            _rh_rd(net)
        elif algo == "rd":
            _rd(net)
        elif algo == "binomial":
            _binomial(net)
        elif algo == "ahc":
            _ahc(net, list(groups) if groups else [P])
        elif algo == "chain":
            if knob < 1:
                raise ValueError("the chain needs m >= 1 pieces")
            _chain(net, knob)
        else:
            raise ValueError(f"unknown algorithm {algo!r}")
        out, stats = net.buf, net.stats()
    if symbolic:
        stats["algebra"] = alg
        res = out
    else:
        res = np.stack([alg.store(alg.finish(out[p], P)) for p in range(P)])
    if squeeze:
        res = res[:, 0, :]
    return (res, stats) if return_stats else res


# --------------------------------------------------------------------------
# the two halves: reduce-scatter and all-gather
# --------------------------------------------------------------------------
HALF_ALGOS = ("direct", "ring", "rh_rd", "generalized", "generalized_xor")


def _ring_rs(net: Net):
    """Ring reduce-scatter with rank q ending on part q (the convention of a
    reduce-scatter that hands rank q block q; all-reduce blog page, "The APIs",
    FSDP/ZeRO paragraph). It is the ring's first phase ("The ring algorithm")
    with the part labels rotated by one: in step t rank r passes part
    (r - t - 1) mod P to r + 1, so part q travels q+1, q+2, ..., q and is
    complete on arrival at q."""
    P = net.P
    parts = partition(net.n, P)
    for t in range(P - 1):
        net.step([(r, (r + 1) % P, *parts[(r - t - 1) % P], REDUCE) for r in range(P)])


def _ring_ag(net: Net):
    """Ring all-gather from rank q holding part q: in step t rank r passes part
    (r - t) mod P (its own part first, then the one it just received)."""
    P = net.P
    parts = partition(net.n, P)
    for t in range(P - 1):
        net.step([(r, (r + 1) % P, *parts[(r - t) % P], COPY) for r in range(P)])


def _direct_rs(net: Net):
    """The one-root schedule's reduce half (rank 0 folds ranks 1..P-1 in rank
    order), then one step in which rank 0 hands part q to rank q."""
    P, n = net.P, net.n
    parts = partition(n, P)
    for s in range(1, P):
        net.step([(s, 0, 0, n, REDUCE)])
    net.step([(0, q, *parts[q], COPY) for q in range(1, P)])


def _direct_ag(net: Net):
    """One step in which every rank q sends part q to every other rank."""
    P = net.P
    parts = partition(net.n, P)
    net.step([(q, d, *parts[q], COPY) for q in range(P) for d in range(P) if d != q])


def _half_input(x, alg, symbolic, P):
    x = np.asarray(x)
    squeeze = x.ndim == 2
    if squeeze:
        x = x[:, None, :]
    if symbolic:
        xacc = np.empty(x.shape, dtype=object)
        for p in range(P):
            xacc[p] = p
    else:
        xacc = np.stack([alg.load(x[p]) for p in range(P)])
    return xacc, squeeze


def reduce_scatter(x: np.ndarray, algo: str, dtype: str, op: str = "sum", n: int | None = None, idx=None,
                   symbolic: bool = False, return_stats: bool = False, steps: int | None = None, factors=None):
    """Replay a reduce-scatter: rank q ends with the reduced part q of the ceil
    split into P parts. x as for ``allreduce``. Returns the result vector
    (element e as rank e // ceil(n / P) holds it), shape (m,) or (B, m).

    Schedules: ring (above), rh_rd = the halving half (P a power of two),
    generalized / generalized_xor = the reduction phase with r = 0, direct =
    one-root fold then hand-out."""
    P = np.asarray(x).shape[0]
    alg = Symbolic(P) if symbolic else Algebra(dtype, op)
    xacc, squeeze = _half_input(x, alg, symbolic, P)
    m = xacc.shape[2]
    n = m if n is None else n
    idx = np.arange(n, dtype=np.int64) if idx is None else np.asarray(idx, dtype=np.int64)
    c = -(-n // P) if n else 1
    owner = idx // c
    if P == 1 or n == 0:
        res, stats = xacc[0].copy(), dict(steps=0)
    elif algo in ("generalized", "generalized_xor"):
        grp = tuple(factors) if factors and algo == "generalized" else ("cyclic" if algo == "generalized" else "xor")
        res, stats = _generalized(alg, xacc, n, idx, 0, grp, "reduce", steps if algo == "generalized" else None)
    else:
        net = Net(alg, xacc.copy(), n, idx)
        if algo == "ring":
            _ring_rs(net)
        elif algo == "rh_rd":
            if P & (P - 1):
                raise ValueError("the halving reduce-scatter needs P to be a power of two")
            _halving(net, P)
        elif algo == "direct":
            _direct_rs(net)
        else:
            raise ValueError(f"no reduce-scatter for {algo!r}")
        res = net.buf[owner, :, np.arange(m)].T if m else net.buf[0, :, :0]
        stats = net.stats()
    if symbolic:
        stats["algebra"] = alg
    else:
        res = alg.store(alg.finish(res, P))
    if squeeze:
        res = res[0]
    return (res, stats) if return_stats else res


def all_gather(x: np.ndarray, algo: str, dtype: str, n: int | None = None, idx=None, return_stats: bool = False,
               steps: int | None = None, factors=None):
    """Replay an all-gather: rank q contributes part q of its buffer (the rest
    of its input is ignored); every rank ends with every part. Returns the
    per-rank buffers in x's shape. Pure copies: the bits are the owners'."""
    P = np.asarray(x).shape[0]
    alg = Algebra(dtype, "sum")
    xacc, squeeze = _half_input(x, alg, False, P)
    m = xacc.shape[2]
    n = m if n is None else n
    idx = np.arange(n, dtype=np.int64) if idx is None else np.asarray(idx, dtype=np.int64)
    if P == 1 or n == 0:
        out, stats = xacc.copy(), dict(steps=0)
    elif algo in ("generalized", "generalized_xor"):
        grp = tuple(factors) if factors and algo == "generalized" else ("cyclic" if algo == "generalized" else "xor")
        out, stats = _generalized(alg, xacc, n, idx, 0, grp, "gather", steps if algo == "generalized" else None)
    else:
        net = Net(alg, xacc.copy(), n, idx)
        if algo == "ring":
            _ring_ag(net)
        elif algo == "rh_rd":
            if P & (P - 1):
                raise ValueError("the doubling all-gather needs P to be a power of two")
            _doubling(net, P)
        elif algo == "direct":
            _direct_ag(net)
        else:
            raise ValueError(f"no all-gather for {algo!r}")
        out, stats = net.buf, net.stats()
    res = np.stack([alg.store(out[p]) for p in range(P)])
    if squeeze:
        res = res[:, 0, :]
    return (res, stats) if return_stats else res
