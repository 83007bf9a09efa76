"""Test-only CPU interpreters for what the library exports.

* ``run_table`` executes an exported step table (ar_oprec records) on host
  arrays with snapshot step semantics and workspace slots.
* ``run_fused`` evaluates an exported fused replay program (per range: result
  trees in postfix order, then their destination ranks).

They are generic: they know nothing about any particular schedule. Neither is
the oracle; tests compare their bits with the oracle's.
"""
from __future__ import annotations

import numpy as np


def _widen(bits):
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32)


def _narrow(f):
    u = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def _combine(a, b, dtype, op):
    if op in ("sum", "avg"):
        return a + b
    if dtype == "int32":
        return np.where(b.view(np.int32) > a.view(np.int32), b, a)
    ka = a.view(np.int32) ^ ((a.view(np.int32) >> 31) & 0x7FFFFFFF)
    kb = b.view(np.int32) ^ ((b.view(np.int32) >> 31) & 0x7FFFFFFF)
    return np.where(kb > ka, b, a)


def _to_acc(x, dtype):
    if dtype == "int32":
        return np.asarray(x, dtype=np.int32).view(np.uint32).copy()
    if dtype == "fp32":
        return np.asarray(x, dtype=np.float32).copy()
    return _widen(np.asarray(x, dtype=np.uint16))


def _from_acc(a, dtype):
    if dtype == "int32":
        return a.view(np.int32).copy()
    if dtype == "fp32":
        return a.copy()
    return _narrow(a)


def run_table(x, ops, dtype, op, n, batch=1, nslots=None):
    """x: (P, batch * n) caller buffers. Returns the final caller buffers.

    op "avg": a combination whose result covers all P ranks (counted per
    element alongside the values) is divided by P before it is stored."""
    P = x.shape[0]
    if nslots is None:
        nslots = 1 + max([0] + [max(o.src_slot, o.dst_slot, o.own_slot) for o in ops])
    # slot 0 in the storage dtype; workspace slots in the accumulation type
    user = [np.array(x[p]) for p in range(P)]
    acc_t = np.uint32 if dtype == "int32" else np.float32
    ws = [[np.zeros(batch * n, dtype=acc_t) for _ in range(nslots)] for _ in range(P)]
    cnt = [[np.ones(batch * n, dtype=np.int64) if s == 0 else np.zeros(batch * n, dtype=np.int64)
            for s in range(nslots)] for _ in range(P)]

    def rd(rank, slot, sl):
        if slot == 0:
            return _to_acc(user[rank][sl], dtype)
        return ws[rank][slot][sl].copy()

    def wr(rank, slot, sl, v):
        if slot == 0:
            user[rank][sl] = _from_acc(v, dtype)
        else:
            ws[rank][slot][sl] = v

    def spans(o):
        if batch > 1 and o.offset == 0 and o.length == n:
            return [slice(0, batch * n)]
        return [slice(b * n + o.offset, b * n + o.offset + o.length) for b in range(batch)]

    i = 0
    while i < len(ops):
        j = i
        while j < len(ops) and ops[j].step == ops[i].step:
            j += 1
        pending = []
        for o in ops[i:j]:
            for sl in spans(o):
                s = rd(o.src_rank, o.src_slot, sl)
                c = cnt[o.src_rank][o.src_slot][sl].copy()
                if o.kind == 0:
                    v = _combine(rd(o.dst_rank, o.own_slot, sl), s, dtype, op)
                    c = c + cnt[o.dst_rank][o.own_slot][sl]
                    if op == "avg":
                        v = np.where(c == P, v / np.float32(P), v).astype(np.float32)
                else:
                    v = s
                pending.append((o.dst_rank, o.dst_slot, sl, v, c))
        for rank, slot, sl, v, c in pending:
            wr(rank, slot, sl, v)
            cnt[rank][slot][sl] = c
        i = j
    return np.stack(user)


def run_fused(x, starts, lens, offs, words, dtype, op, n, batch=1):
    """Evaluate an exported fused program on host arrays."""
    P = x.shape[0]
    out = np.array(x)
    acc = [_to_acc(x[p], dtype) for p in range(P)]
    for b in range(batch):
        for st, ln, off in zip(starts, lens, offs):
            sl = slice(b * n + st, b * n + st + ln)
            w = off
            ntrees = words[w]
            w += 1
            for _ in range(ntrees):
                nl, no = words[w], words[w + 1]
                leaves = words[w + 2: w + 2 + nl]
                ncomb = words[w + 2 + nl: w + 2 + 2 * nl]
                outs = words[w + 2 + 2 * nl: w + 2 + 2 * nl + no]
                stack = []
                for leaf, c in zip(leaves, ncomb):
                    stack.append(acc[leaf][sl])
                    for _ in range(c):
                        top = stack.pop()
                        below = stack.pop()
                        stack.append(_combine(below, top, dtype, op))
                assert len(stack) == 1
                res = stack[0] / np.float32(P) if op == "avg" else stack[0]
                for r in outs:
                    out[r][sl] = _from_acc(res, dtype)
                w += 2 + 2 * nl + no
    return out


def dag_parse(words, off=0):
    """One serialized DAG program at words[off:]: (S, leaves, level starts,
    instructions as (dst, a, b), outputs as (slot, rank))."""
    S, nleaf, nlev, ninstr, nout = words[off: off + 5]
    p = off + 5
    leaves = list(words[p: p + nleaf])
    p += nleaf
    lv = list(words[p: p + nlev + 1])
    p += nlev + 1
    ins = [(w & 1023, (w >> 10) & 1023, (w >> 20) & 1023) for w in words[p: p + ninstr]]
    p += ninstr
    outs = [(w >> 16, w & 0xFFFF) for w in words[p: p + nout]]
    return S, leaves, lv, ins, outs


def dag_hazards(prog):
    """Every level's combinations must be independent when lanes of different
    threads run them in any order: distinct destination slots, and no slot one
    combination writes is read by another combination of the same level."""
    S, leaves, lv, ins, outs = prog
    for l in range(len(lv) - 1):
        level = ins[lv[l]: lv[l + 1]]
        dsts = [d for d, _, _ in level]
        assert len(set(dsts)) == len(dsts), ("duplicate destination", l)
        for i, (d, _, _) in enumerate(level):
            for j, (_, a, b) in enumerate(level):
                assert j == i or d not in (a, b), ("read and written in one level", l, d)
        assert all(max(d, a, b) < S for d, a, b in level)
    assert all(s < S for s, _ in outs)


def run_dag(x, starts, lens, shared, offs, maps, words, dtype, op, n, batch=1):
    """Evaluate exported DAG programs on host arrays: per range its own program,
    or (shared) the one program with leaf and output ranks renamed by the
    range's row of maps. Levels run their combinations in reverse order, so a
    hazard that dag_hazards misses would show as wrong values."""
    P = x.shape[0]
    out = np.array(x)
    acc = [_to_acc(x[p], dtype) for p in range(P)]
    for r, (st, ln) in enumerate(zip(starts, lens)):
        prog = dag_parse(words, 0 if shared else offs[r])
        dag_hazards(prog)
        S, leaves, lv, ins, outs = prog
        ren = (lambda q: int(maps[r][q])) if shared else (lambda q: q)
        for b in range(batch):
            sl = slice(b * n + st, b * n + st + ln)
            vals = [None] * S
            for k, q in enumerate(leaves):
                vals[k] = acc[ren(q)][sl].copy()
            for l in range(len(lv) - 1):
                for d, a, bb in reversed(ins[lv[l]: lv[l + 1]]):
                    vals[d] = _combine(vals[a], vals[bb], dtype, op)
            for s, q in outs:
                res = vals[s] / np.float32(P) if op == "avg" else vals[s]
                out[ren(q)][sl] = _from_acc(res, dtype)
    return out
