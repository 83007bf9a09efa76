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
"""
from __future__ import annotations

import math

from .numerics import ceil_log2


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
