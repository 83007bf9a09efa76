"""Cost-model arithmetic stated by the pages (oracle).

* Per-message cost alpha + bytes * beta, plus gamma per combined element
  (generalized-Allreduce paper, cost-model paragraph after Fig. 1, after Chan
  et al.; the formula itself is missing from the extracted text, so this is
  the reading: one step costs alpha + (data sent by the busiest rank) * beta +
  (elements combined by the busiest rank) * gamma, with u = m / P).
* Closed forms the paper states in prose: the straightforward/ring cost
  (eqs. (15)-(16): 2(P-1) steps, 2(P-1)u sent, (P-1)u combined), the
  bandwidth-optimal cost (eq. (25): same data in 2 ceil(log P) steps) and the
  intermediate cost (eq. (36)): 2L - r steps, (2^r - 1) L u extra data sent
  and at worst (2^r - 1)(2L - 2) u extra combinations.
* algbw / busbw and the worked estimate of the all-reduce blog page
  ("Reading benchmarks: algbw and busbw", "Worked example").
* The pipelined chain reduce of the "Reduction Operator" page (p + m - 2
  steps of n / m bytes; optimal segment count).
* Model-driven choice of schedule: the generalized-Allreduce paper picks its
  step count r by minimising eq. (36) under measured alpha, beta, gamma
  ("Intermediate version", eq. (37), experiments section); the all-reduce blog
  page's library picks an algorithm per call from a tuning model ("Protocols:
  Simple, LL and LL128"). ``select`` enumerates every schedule the oracle
  replays and evaluates the model on the exact per-step, per-rank element
  counts of the replay (not on the prose closed forms, which hold for P | n
  and state the combine count only as a worst case).
"""
from __future__ import annotations

import math

import numpy as np

from . import schedules
from .numerics import ceil_log2

ELT_BYTES = {"int32": 4, "fp32": 4, "bf16": 2}


def message_time(nbytes: float, alpha: float, bandwidth: float) -> float:
    """Blog page cost model: a message of n bytes over one link costs alpha + n / B."""
    return alpha + nbytes / bandwidth


def ring_time(P: int, m: float, alpha: float, beta: float, gamma: float) -> float:
    u = m / P
    return 2 * (P - 1) * alpha + 2 * (P - 1) * u * beta + (P - 1) * u * gamma


def bandwidth_optimal_time(P: int, m: float, alpha: float, beta: float, gamma: float) -> float:
    u = m / P
    L = ceil_log2(P)
    return 2 * L * alpha + 2 * (P - 1) * u * beta + (P - 1) * u * gamma


def intermediate_time(P: int, m: float, r: int, alpha: float, beta: float, gamma: float) -> float:
    """Prose form of eq. (36), valid for 0 <= r < ceil(log P)."""
    u = m / P
    L = ceil_log2(P)
    extra = (1 << r) - 1
    return ((2 * L - r) * alpha + (2 * (P - 1) + extra * L) * u * beta
            + ((P - 1) + extra * (2 * L - 2)) * u * gamma)


def optimal_r(P: int, m: float, alpha: float, beta: float, gamma: float) -> int:
    """Eq. (37) is missing from the text; enumerate the integer r that minimises (36)."""
    L = ceil_log2(P)
    best = min(range(L), key=lambda r: intermediate_time(P, m, r, alpha, beta, gamma)) if L else 0
    return best


def algbw(size_bytes: float, seconds: float) -> float:
    return size_bytes / seconds


def busbw(algbw_value: float, N: int) -> float:
    """Bus bandwidth = algbw * 2(N-1)/N, the ring's traffic factor."""
    return algbw_value * 2 * (N - 1) / N


def estimated_allreduce_seconds(size_bytes: float, N: int, busbw_value: float) -> float:
    """Blog page's estimate: time = 2(N-1)/N * S / busbw."""
    return 2 * (N - 1) / N * size_bytes / busbw_value


def ring_bytes_per_rank(P: int, S: float) -> float:
    """Each rank sends (and receives) 2(N-1)S/N bytes in the ring."""
    return 2 * (P - 1) * S / P


def pipelined_chain_time(n: float, p: int, m: int, t_start: float, t_byte: float) -> float:
    """'Reduction Operator' page, pipelined reduction: (T_start + n/m T_byte)(p + m - 2)."""
    return (t_start + n / m * t_byte) * (p + m - 2)


def pipelined_chain_best_m(n: float, p: int, t_start: float, t_byte: float) -> float:
    return math.sqrt(n * (p - 2) * t_byte / t_start)


# --------------------------------------------------------------------------
# model-driven choice of schedule
# --------------------------------------------------------------------------
def step_counts(P: int, n: int, algo: str, knob: int = 0, groups=None, coll: str = "allreduce",
                steps: int | None = None):
    """Per-step, per-rank elements sent, received and combined by one instance.

    Counts come from the oracle's own replay of the schedule on a one-offset
    sample (the simulator counts whole-buffer elements whatever the sample).
    Nothing moves when n == 0 or P == 1: zero steps. coll selects the
    Allreduce or its reduce-scatter / all-gather half.
    """
    key = (P, n, algo, knob, tuple(groups) if groups else None, coll, steps)
    if key in _COUNTS:
        return _COUNTS[key]
    z = np.zeros((0, P), dtype=np.int64)
    if P == 1 or n == 0:
        return z, z, z
    x = np.zeros((P, 1), dtype=np.int32)
    if coll == "reduce_scatter":
        _, st = schedules.reduce_scatter(x, algo, "int32", "sum", n=n, idx=[0], return_stats=True, steps=steps)
    elif coll == "all_gather":
        _, st = schedules.all_gather(x, algo, "int32", n=n, idx=[0], return_stats=True, steps=steps)
    else:
        _, st = schedules.allreduce(x, algo, "int32", "sum", knob=knob, groups=groups, n=n, idx=[0],
                                    return_stats=True, steps=steps)
    out = tuple(np.asarray(st[k], dtype=np.int64).reshape(-1, P) for k in ("sent", "recv", "reduced"))
    for a in out:
        a.setflags(write=False)
    if len(_COUNTS) > 4096:
        _COUNTS.clear()
    _COUNTS[key] = out
    return out


_COUNTS: dict = {}  # replays are deterministic: counts per argument tuple are computed once


def model_seconds(counts, elt: int, batch: int, alpha: float, beta: float, gamma: float,
                  form: str = "busiest") -> float:
    """alpha per step + beta per byte moved + gamma per byte combined.

    form "busiest": in each step the busiest rank's bytes (the larger of what
    it sends and receives; what it combines), summed over steps -- every rank
    on its own links, the paper's model. form "all_ranks": every rank's bytes
    summed -- all ranks share one memory.
    """
    sent, recv, red = counts
    S = int(sent.shape[0])
    if form == "busiest":
        xb = int(np.maximum(sent, recv).max(axis=1).sum()) if S else 0
        xg = int(red.max(axis=1).sum()) if S else 0
    elif form == "all_ranks":
        xb, xg = int(sent.sum()), int(red.sum())
    else:
        raise ValueError(form)
    return alpha * S + beta * (float(xb) * elt * batch) + gamma * (float(xg) * elt * batch)


def chain_pieces(P: int, n: int, elt: int, batch: int, alpha: float, beta: float, gamma: float):
    """Piece counts for the pipelined chain: floor and ceiling of the optimum of
    the "Reduction Operator" page's time (T_start + (n/m) T_byte)(p + m - 2),
    taken for the whole Allreduce (the reduce with T_byte = beta + gamma, the
    broadcast with beta): m* = sqrt(M (P - 2)(2 beta + gamma) / (2 alpha)) for M
    bytes per rank, clamped to [1, min(4096, n)]."""
    cap = min(4096, max(1, n))
    M = float(n) * elt * batch
    if P <= 2:
        x = 0.0
    elif alpha > 0:
        x = math.sqrt(M * (P - 2) * (2 * beta + gamma) / (2 * alpha))
    else:
        x = float(cap)
    out = []
    for v in (math.floor(x), math.ceil(x)):
        k = 1 if v < 1 else cap if v > cap else int(v)
        if not out or out[-1] != k:
            out.append(k)
    return out


def candidates(P: int, algo: str = "auto", groups=None, coll: str = "allreduce", steps: int | None = None,
               chain=()):
    """(algo, knob) pairs in tie-breaking order (knob up to the reduction steps;
    ``chain`` the piece counts tried for the pipelined chain)."""
    L = ceil_log2(P) if not steps else steps
    pow2 = P & (P - 1) == 0
    if algo == "chain":
        return [("chain", m) for m in chain]
    if coll != "allreduce":
        if algo != "auto":
            return [(algo, 0)]
        out = [("direct", 0), ("ring", 0)] + ([("rh_rd", 0)] if pow2 else []) + [("generalized", 0)]
        return out + ([("generalized_xor", 0)] if pow2 else [])
    if algo != "auto":
        return [(algo, r) for r in range(L + 1)]
    out = [(a, 0) for a in ("direct", "ring", "rh_rd", "rd", "binomial")]
    out += [("generalized", r) for r in range(L + 1)]
    if P & (P - 1) == 0:
        out += [("generalized_xor", r) for r in range(L + 1)]
    if groups:
        out.append(("ahc", 0))
    return out + [("chain", m) for m in chain]


def select(P: int, n: int, dtype: str, alpha: float, beta: float, gamma: float, form: str = "busiest",
           algo: str = "auto", batch: int = 1, groups=None, coll: str = "allreduce", steps: int | None = None):
    """(algo, knob, seconds) of least model time; ties: fewer steps, then earlier candidate.
    ``steps`` (the generalized algorithm's reduction steps) applies to an explicit algorithm only."""
    best = None
    steps = steps if algo != "auto" else None
    chain = chain_pieces(P, n, ELT_BYTES[dtype], batch, alpha, beta, gamma) if coll == "allreduce" else ()
    for a, r in candidates(P, algo, groups, coll, steps, chain):
        c = step_counts(P, n, a, r, groups if a == "ahc" else None, coll, steps)
        t = model_seconds(c, ELT_BYTES[dtype], batch, alpha, beta, gamma, form)
        key = (t, c[0].shape[0])
        if best is None or key < best[0]:
            best = (key, a, r)
    return best[1], best[2], best[0][0]
