"""Seeded synthetic rank buffers for the Allreduce workloads.

This module is the only code shared by the CPU oracle and the HIP path. It
draws random numbers and lays them out; it holds none of the Allreduce
arithmetic. Every draw is rank-major from ``numpy.random.default_rng(seed)``,
so the same (workload, seed) always gives the same arrays on any machine.

Workloads (P ranks, each rank one buffer of n elements):

* ``ring_int32``     P=5, n=4096 int32, uniform integers in [-2^20, 2^20]
* ``rh_fp32``        P=8, n=2^20 fp32, N(0, 1)
* ``prime_fp32``     P=7, n=2^24 fp32, N(0, sigma=1e-3) ("gradient-like")
* ``small_batch``    P in {3, 6, 12, 24}, 10^4 instances x 106 fp32, U(-1, 1)
* ``ahc_bf16``       P=192 in groups (64, 128), n=2^20 bf16 rounded from N(0, 1)

The 106-fp32 instances (424 B) stand in for the production average message
of about 425 bytes that the generalized-Allreduce paper quotes in its
introduction; no dataset is involved anywhere.

bf16 buffers are returned as ``uint16`` bit patterns. The fp32 -> bf16 step
here is part of the input recipe (draw fp32, round to nearest even), not of
the method.
"""
from __future__ import annotations

import numpy as np

BF16 = "bf16"
FP32 = "fp32"
INT32 = "int32"

WORKLOADS = {
    # name: (P, n, dtype, groups, batch, inst_len)
    "ring_int32": dict(P=5, n=4096, dtype=INT32),
    "rh_fp32": dict(P=8, n=1 << 20, dtype=FP32),
    "prime_fp32": dict(P=7, n=1 << 24, dtype=FP32),
    "small_batch": dict(P=24, n=10_000 * 106, dtype=FP32, batch=10_000, inst_len=106),
    "ahc_bf16": dict(P=192, n=1 << 20, dtype=BF16, groups=(64, 128)),
}


def fp32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bits.

    Input values must be finite (the generators below only make finite values).
    """
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = u + np.uint32(0x7FFF) + lsb
    return (rounded >> np.uint32(16)).astype(np.uint16)


def bf16_bits_to_fp32(b: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    return (np.asarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def uniform_int32(P: int, n: int, seed: int = 0, lo: int = -(1 << 20), hi: int = 1 << 20) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi, size=(P, n), endpoint=True, dtype=np.int64).astype(np.int32)


def normal_fp32(P: int, n: int, seed: int = 0, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((P, n), dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return x


def uniform_fp32(P: int, n: int, seed: int = 0, lo: float = -1.0, hi: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.uniform(lo, hi, size=(P, n)).astype(np.float32)


def normal_bf16(P: int, n: int, seed: int = 0) -> np.ndarray:
    return fp32_to_bf16_bits(normal_fp32(P, n, seed))


def make(dtype: str, P: int, n: int, seed: int = 0, dist: str | None = None) -> np.ndarray:
    """Rank-major (P, n) array for ``dtype`` with the workload's default distribution.

    dist: None picks the default for the dtype (int32 -> uniform integers in
    [-2^20, 2^20], fp32 -> N(0,1), bf16 -> N(0,1) rounded). Other choices:
    "normal_1e-3", "uniform_pm1", "small_int" (integers in [-8, 8], exact in
    bf16 and fp32 so every summation order agrees).
    """
    if dist is None:
        dist = {INT32: "int", FP32: "normal", BF16: "normal"}[dtype]
    if dist == "small_int":
        rng = np.random.default_rng(seed)
        v = rng.integers(-8, 8, size=(P, n), endpoint=True).astype(np.float32)
        if dtype == INT32:
            return v.astype(np.int32)
        return fp32_to_bf16_bits(v) if dtype == BF16 else v
    if dtype == INT32:
        return uniform_int32(P, n, seed)
    if dist == "normal":
        v = normal_fp32(P, n, seed)
    elif dist == "normal_1e-3":
        v = normal_fp32(P, n, seed, sigma=1e-3)
    elif dist == "uniform_pm1":
        v = uniform_fp32(P, n, seed)
    else:
        raise ValueError(f"unknown distribution {dist!r}")
    return fp32_to_bf16_bits(v) if dtype == BF16 else v


def workload(name: str, seed: int = 0, P: int | None = None) -> np.ndarray:
    """Inputs for one named workload (``small_batch`` takes P in {3, 6, 12, 24})."""
    w = WORKLOADS[name]
    if name == "ring_int32":
        return uniform_int32(w["P"], w["n"], seed)
    if name == "rh_fp32":
        return normal_fp32(w["P"], w["n"], seed)
    if name == "prime_fp32":
        return normal_fp32(w["P"], w["n"], seed, sigma=1e-3)
    if name == "small_batch":
        return uniform_fp32(P if P is not None else w["P"], w["n"], seed)
    if name == "ahc_bf16":
        return normal_bf16(w["P"], w["n"], seed)
    raise KeyError(name)


def sample_indices(n: int, parts: int, count: int = 4096, seed: int = 1) -> np.ndarray:
    """Sorted element indices for sampled checks at full size.

    Mixes uniformly drawn indices with every boundary of an equal-ceil split of
    [0, n) into ``parts`` pieces (and its neighbours), so ragged part edges are
    always covered.
    """
    rng = np.random.default_rng(seed)
    picks = [rng.integers(0, n, size=min(count, n))] if n else []
    if n and parts:
        c = -(-n // parts)
        edges = np.arange(0, parts + 1, dtype=np.int64) * c
        for d in (-2, -1, 0, 1):
            picks.append(np.clip(edges + d, 0, n - 1))
        picks.append(np.array([0, n - 1]))
    if not picks:
        return np.zeros(0, dtype=np.int64)
    return np.unique(np.concatenate(picks).astype(np.int64))


# ---------------------------------------------------------------------------
# counter-based values for buffers too large to draw and ship from the host
# ---------------------------------------------------------------------------
_M1, _M2 = 65521, 65519  # the two largest primes below 2^16


def counter_ints(p: int, e, seed: int = 0):
    """Value of rank p at element offsets e (int64 array, NumPy or torch):
    with a = e mod 65521 and b = e mod 65519,
    (a b + 7 a + 3 b + 11 p + seed) mod 4093 - 2046, an integer in [-2046, 2046].

    A pure function of (seed, p, e), so the GPU can fill a buffer of any size
    chunk by chunk and the host can compute any sampled offset on its own. The
    pattern repeats only after 65521 * 65519 (about 2^32) offsets, and small
    integers keep fp32 sums of a few ranks exact in any order.
    """
    a, b = e % _M1, e % _M2
    return (a * b + 7 * a + 3 * b + 11 * p + seed) % 4093 - 2046


def fill_counter_fp32(row, p: int, seed: int = 0, chunk: int = 1 << 27) -> None:
    """Fill a 1-D float32 torch tensor (any device) with counter_ints(p, 0..len-1)."""
    import torch
    n = row.numel()
    for s in range(0, n, chunk):
        e = torch.arange(s, min(n, s + chunk), dtype=torch.int64, device=row.device)
        row[s: s + e.numel()] = counter_ints(p, e, seed).to(torch.float32)
