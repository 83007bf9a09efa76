"""Helpers for GPU tests: move seeded host arrays into per-rank device buffers,
call the library through its C ABI, and bring the results back."""
from __future__ import annotations

import numpy as np

import allreduce_schedule_algorithms_amd as A


def torch_mod():
    import torch
    return torch


def to_device(x: np.ndarray, dtype: str, misalign: bool = False):
    """One CUDA tensor per rank holding x[p] (bf16 given as uint16 bits).

    misalign=True offsets every buffer by one element inside a larger
    allocation, so the library must take its per-element path.
    """
    torch = torch_mod()
    P = x.shape[0]
    bufs, keep = [], []
    for p in range(P):
        row = np.ascontiguousarray(x[p])
        if dtype == "bf16":
            t = torch.from_numpy(row.view(np.int16)).view(torch.bfloat16)
        else:
            t = torch.from_numpy(row)
        if misalign:
            big = torch.empty(row.size + 8, dtype=t.dtype, device="cuda")
            v = big[1: 1 + row.size]
            v.copy_(t.cuda())
            keep.append(big)
            bufs.append(v)
        else:
            bufs.append(t.cuda())
    return bufs, keep


def from_device(bufs, dtype: str) -> np.ndarray:
    torch = torch_mod()
    out = []
    for t in bufs:
        if dtype == "bf16":
            out.append(t.view(torch.int16).cpu().numpy().view(np.uint16))
        else:
            out.append(t.cpu().numpy())
    return np.stack(out)


def gpu_allreduce(x: np.ndarray, algo: str, dtype: str, op: str = "sum", knob: int = 0, exec: str = "fused",
                  groups=None, batch: int = 1, misalign: bool = False, stream=None,
                  collective: str = "allreduce", steps: int = 0) -> np.ndarray:
    """Run one collective on cuda:0 through ar_allreduce_ex and return every rank's buffer."""
    torch = torch_mod()
    P, total = x.shape
    n = total // batch
    bufs, keep = to_device(x, dtype, misalign)
    call = A.make_call(P, n, dtype, op, algo, knob, exec, batch, groups, collective=collective, steps=steps)
    s = stream if stream is not None else torch.cuda.current_stream()
    A.ar_allreduce_ex([b.data_ptr() for b in bufs], call, s)
    torch.cuda.synchronize()
    out = from_device(bufs, dtype)
    del keep
    return out


def bits(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a)
    return a.view(np.uint16) if a.dtype == np.uint16 else a.view(np.uint32)
