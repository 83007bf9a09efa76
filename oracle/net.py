"""A P-rank message simulator with snapshot step semantics (oracle).

Ranks are simulated in one process, the way the all-reduce blog page runs its
ring on Python lists ("The ring algorithm"): in every step all messages are
first read from the pre-step state, then applied. A message carries the
elements [lo, hi) of the sender's buffer to the receiver, which either adds
them into its own copy of the same elements (REDUCE) or overwrites its copy
(COPY). Every schedule here only ever exchanges elements at the same offset
in every rank's buffer (the generalized-Allreduce paper's data matrix has
one element index per row, across all processes), so [lo, hi) is the same
range at sender and receiver.

The simulator can run on a sample of element offsets: ``idx`` lists the
global offsets that are kept (sorted). A message over [lo, hi) then touches
the sampled offsets inside that range only. Because elements never move
between offsets, the values at the kept offsets are exactly those of a run
over the whole buffer.

Traffic counters are kept in elements of the full (unsampled) buffer, per
instance.
"""
from __future__ import annotations

import numpy as np

REDUCE = "reduce"
COPY = "copy"


def partition(n: int, C: int) -> list[tuple[int, int]]:
    """Split [0, n) into C parts of ceil(n / C) elements; the last ones may be short or empty.

    This is the chunking rule of the blog page's ring simulation: chunk size
    is the ceiling of n / C and chunk k covers [k c, (k + 1) c) clipped to n.
    """
    c = -(-n // C) if C > 0 else 0
    return [(min(k * c, n), min((k + 1) * c, n)) for k in range(C)]


class Net:
    def __init__(self, algebra, x_acc: np.ndarray, n: int, idx: np.ndarray):
        # x_acc: (P, B, m) accumulation arrays, m = len(idx)
        self.alg = algebra
        self.buf = x_acc
        self.P = x_acc.shape[0]
        self.n = n
        self.idx = np.asarray(idx, dtype=np.int64)
        self.nsteps = 0
        self.sent: list[np.ndarray] = []     # per step: elements sent by each rank
        self.recv: list[np.ndarray] = []     # per step: elements received by each rank
        self.reduced: list[np.ndarray] = []  # per step: elements combined at each rank
        self.peers: list[list[tuple[int, int]]] = []  # per step: (src, dst) pairs

    def _span(self, lo: int, hi: int) -> slice:
        a = int(np.searchsorted(self.idx, lo, side="left"))
        b = int(np.searchsorted(self.idx, hi, side="left"))
        return slice(a, b)

    def step(self, msgs):
        """Run one step: msgs is a list of (src, dst, lo, hi, kind)."""
        sent = np.zeros(self.P, dtype=np.int64)
        recv = np.zeros(self.P, dtype=np.int64)
        red = np.zeros(self.P, dtype=np.int64)
        staged = []
        for src, dst, lo, hi, kind in msgs:
            if src == dst:
                raise ValueError("a rank does not send to itself")
            sl = self._span(lo, hi)
            staged.append((dst, sl, kind, self.buf[src, :, sl].copy()))
            sent[src] += hi - lo
            recv[dst] += hi - lo
            if kind == REDUCE:
                red[dst] += hi - lo
        for dst, sl, kind, data in staged:
            if kind == REDUCE:
                self.buf[dst, :, sl] = self.alg.op(self.buf[dst, :, sl], data)
            elif kind == COPY:
                self.buf[dst, :, sl] = data
            else:
                raise ValueError(kind)
        self.nsteps += 1
        self.sent.append(sent)
        self.recv.append(recv)
        self.reduced.append(red)
        self.peers.append([(m[0], m[1]) for m in msgs if m[3] > m[2]])

    def stats(self) -> dict:
        z = np.zeros((0, self.P), dtype=np.int64)
        return dict(
            steps=self.nsteps,
            sent=np.array(self.sent) if self.sent else z,
            recv=np.array(self.recv) if self.recv else z,
            reduced=np.array(self.reduced) if self.reduced else z,
            peers=self.peers,
        )
