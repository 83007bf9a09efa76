"""Reduction algebras, fp64 reference and error bounds (oracle).

The elementwise vector operator is the one the "Reduction Operator" page
defines for its binomial-tree reduce (each output element combines the two
input elements at the same index). The precision rules are the reading of the
"Numerics and reproducibility" section of the all-reduce blog page: bf16
values are summed with fp32 partials and rounded to bf16 once, when a part's
reduction is complete; fp32 is summed in fp32 with round-to-nearest-even;
int32 sums wrap modulo 2^32.

An ``Algebra`` turns a rank buffer into the accumulation representation
(``load``), combines two accumulation arrays (``op``) and turns a finished
value back into the storage dtype (``store``). Because the only rounding in
bf16 mode happens on a complete value and a copy of a rounded value is the
rounded copy, ``store`` may be applied once at the very end of a replay.
"""
from __future__ import annotations

import numpy as np

U32 = np.uint32


# --------------------------------------------------------------------------
# bf16 helpers (the oracle's own; the input generator has a separate one)
# --------------------------------------------------------------------------
def bf16_to_f32(bits: np.ndarray) -> np.ndarray:
    """bf16 is the top half of an fp32 pattern, so widening is exact."""
    w = np.asarray(bits, dtype=np.uint16).astype(U32)
    return (w * U32(65536)).view(np.float32)


def f32_to_bf16(v: np.ndarray) -> np.ndarray:
    """Round finite fp32 values to bf16, nearest with ties to even.

    Keep the upper 16 bits; the dropped lower half decides: above the halfway
    point 0x8000 round up, below round down, exactly halfway round to the even
    upper half.
    """
    u = np.ascontiguousarray(v, dtype=np.float32).view(U32)
    upper = u // U32(65536)
    lower = u % U32(65536)
    up = (lower > U32(0x8000)) | ((lower == U32(0x8000)) & (upper % U32(2) == U32(1)))
    return (upper + up.astype(U32)).astype(np.uint16)


def max_total(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """Elementwise maximum under the total order of non-NaN floats with -0 < +0."""
    take_b = (b > a) | ((b == a) & np.signbit(a) & ~np.signbit(b))
    return np.where(take_b, b, a)


class Algebra:
    """Accumulation semantics for one (dtype, op) pair."""

    def __init__(self, dtype: str, op: str):
        if dtype not in ("int32", "fp32", "bf16"):
            raise ValueError(dtype)
        if op not in ("sum", "max", "avg"):
            raise ValueError(op)
        if op == "avg" and dtype == "int32":
            raise ValueError("avg is defined for floating-point data only")
        self.dtype, self.opname = dtype, op

    def load(self, x: np.ndarray) -> np.ndarray:
        if self.dtype == "int32":
            a = np.asarray(x, dtype=np.int32)
            return a.view(U32).copy() if self.opname == "sum" else a.copy()
        if self.dtype == "fp32":
            return np.asarray(x, dtype=np.float32).copy()
        return bf16_to_f32(x)

    def op(self, a: np.ndarray, b: np.ndarray) -> np.ndarray:
        if self.opname in ("sum", "avg"):
            return a + b  # uint32 wraps, float32 rounds to nearest even
        if self.dtype == "int32":
            return np.maximum(a, b)
        return max_total(a, b)

    def finish(self, acc: np.ndarray, P: int) -> np.ndarray:
        """avg: the complete sum divided by P once, in the accumulation type
        (all-reduce blog page, "The APIs": the average is taken inside the
        collective). Reading: one IEEE division of the finished sum, no
        pre-scaling; other ops pass through."""
        if self.opname != "avg":
            return acc
        return (np.asarray(acc, dtype=np.float32) / np.float32(P)).astype(np.float32)

    def store(self, acc: np.ndarray) -> np.ndarray:
        if self.dtype == "int32":
            return acc.view(np.int32) if acc.dtype == U32 else acc.astype(np.int32)
        if self.dtype == "fp32":
            return acc.astype(np.float32)
        return f32_to_bf16(acc)


class Symbolic:
    """Tree algebra: values are interned node ids of commutative expression trees.

    Leaves are 0..P-1 (rank ids); an internal node is the unordered pair of its
    children, so two trees that differ only by swapping operands of one
    combination get the same id (every operator here is commutative bitwise).
    """

    def __init__(self, P: int):
        self.P = P
        self._ids: dict = {}
        self._kids: list = []

    def node(self, a: int, b: int) -> int:
        key = (a, b) if a <= b else (b, a)
        nid = self._ids.get(key)
        if nid is None:
            nid = self.P + len(self._kids)
            self._ids[key] = nid
            self._kids.append(key)
        return nid

    def op(self, a: np.ndarray, b: np.ndarray) -> np.ndarray:
        f = np.frompyfunc(self.node, 2, 1)
        return np.asarray(f(a, b), dtype=object)

    def load(self, x: np.ndarray) -> np.ndarray:
        return np.asarray(x, dtype=object).copy()

    def finish(self, acc: np.ndarray, P: int) -> np.ndarray:
        return acc  # trees: the division does not change the combination order

    def store(self, acc: np.ndarray) -> np.ndarray:
        return acc

    def children(self, nid: int):
        return None if nid < self.P else self._kids[nid - self.P]

    def leaves(self, nid: int) -> list:
        out, stack = [], [int(nid)]
        while stack:
            v = stack.pop()
            k = self.children(v)
            if k is None:
                out.append(v)
            else:
                stack.extend(k)
        return sorted(out)

    def show(self, nid: int) -> str:
        k = self.children(int(nid))
        if k is None:
            return f"x{int(nid)}"
        a, b = sorted((self.show(k[0]), self.show(k[1])))
        return f"({a}+{b})"

    def depth(self, nid: int) -> int:
        k = self.children(int(nid))
        return 0 if k is None else 1 + max(self.depth(k[0]), self.depth(k[1]))


# --------------------------------------------------------------------------
# references and bounds
# --------------------------------------------------------------------------
def brute_force(x: np.ndarray, dtype: str, op: str) -> np.ndarray:
    """The plain Allreduce result for int32 sum (mod 2^32) and max: order-free and exact."""
    if op == "max":
        if dtype == "int32":
            return np.max(np.asarray(x, dtype=np.int32), axis=0)
        v = bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)
        r = v[0]
        for p in range(1, v.shape[0]):
            r = max_total(r, v[p])
        return f32_to_bf16(r) if dtype == "bf16" else r
    if dtype == "int32":
        s = np.asarray(x, dtype=np.int64).sum(axis=0)
        return (s % (1 << 32)).astype(np.uint64).astype(np.uint32).view(np.int32)
    raise ValueError("floating-point sums depend on the schedule; use fp64_reference")


def fp64_reference(x: np.ndarray, dtype: str) -> np.ndarray:
    """fp64 sum of the exactly widened inputs (the comparison point for fp sums)."""
    v = bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)
    return v.astype(np.float64).sum(axis=0)


def sum_error_bound(x: np.ndarray, dtype: str) -> np.ndarray:
    """Elementwise bound on |schedule result - exact sum| for any summation tree.

    Any binary tree of P-1 fp32 additions with round-to-nearest has error at
    most gamma_{P-1} * sum|x_p| with gamma_k = k u / (1 - k u), u = 2^-24
    (each leaf passes through at most P-1 roundings). bf16 adds one final
    rounding of relative size at most 2^-8 of the fp32 result.
    """
    v = bf16_to_f32(x) if dtype == "bf16" else np.asarray(x, dtype=np.float32)
    P = v.shape[0]
    u = 2.0 ** -24
    k = max(P - 1, 1)
    gamma = k * u / (1 - k * u)
    absum = np.abs(v.astype(np.float64)).sum(axis=0)
    b = gamma * absum
    if dtype == "bf16":
        b = b + 2.0 ** -8 * (np.abs(v.astype(np.float64).sum(axis=0)) + b)
    return b


def normwise_rel_error(y: np.ndarray, ref: np.ndarray) -> float:
    """max|y - ref| / max|ref| (the normwise tolerance measure)."""
    y64 = np.asarray(y, dtype=np.float64)
    den = float(np.max(np.abs(ref))) if ref.size else 0.0
    num = float(np.max(np.abs(y64 - ref))) if ref.size else 0.0
    return num / den if den > 0 else num


def ceil_log2(P: int) -> int:
    """ceil(log2 P) for P >= 1."""
    return (P - 1).bit_length()
