"""MI355X-native Allreduce schedules: Python side of libar_mi355x.so.

``_ar`` is the ctypes binding of include/ar.h (same function names). The
helpers below only marshal torch tensors into those calls; the product path
has no CPU fallback and fails loudly when the library is missing.
"""
from __future__ import annotations

from . import _ar
from ._ar import (  # noqa: F401
    ALGO_NAMES, ALGOS, AR_KNOB_AUTO, COLLECTIVES, COST_FORMS, DTYPES, EXECS, OPS, Algo, ArError, Collective,
    CostForm, Dtype, Exec, Kernel, Op, Schedule, Status, ar_all_gather, ar_allreduce, ar_allreduce_ex,
    ar_get_cost_model, ar_kernel_of,
    ar_last_error_message, ar_last_hip_error, ar_reduce_scatter, ar_schedule_build, ar_select, ar_set_cost_model,
    ar_set_launch_blocks, ar_status_string, ar_table_check, ar_table_check_ex, ar_version, ar_workspace_bytes,
    make_call, marshal_ptrs, ar_cache_stats_get, ar_release_cached, ar_allreduce_noalloc, AR_NOALLOC_SCRATCH_BYTES,
)

_TORCH_DTYPE = {"int32": "int32", "fp32": "float32", "bf16": "bfloat16"}


def allreduce(tensors, algo="ring", op="sum", knob=0, exec="fused", batch=1, groups=None,
              stream=None, workspace=None, collective="allreduce", steps=0):
    """In-place Allreduce over a list of P equally sized CUDA tensors (one per rank).

    dtype comes from the tensors (int32, float32 or bfloat16); each tensor holds
    ``batch`` contiguous instances. ``stream`` defaults to torch's current stream.
    ``collective`` selects the reduce-scatter or all-gather half instead; ``steps``
    sets the generalized algorithm's reduction steps (0: ceil(log2 P)).
    """
    import torch

    P = len(tensors)
    t0 = tensors[0]
    rev = {v: k for k, v in _TORCH_DTYPE.items()}
    dname = str(t0.dtype).replace("torch.", "")
    if dname not in rev:
        raise ArError(Status.AR_INVALID_ARGUMENT, f"unsupported tensor dtype {t0.dtype}")
    for t in tensors:
        if t.dtype != t0.dtype or t.numel() != t0.numel() or not t.is_cuda or not t.is_contiguous():
            raise ArError(Status.AR_INVALID_ARGUMENT, "tensors must be contiguous CUDA tensors of one dtype and size")
    total = t0.numel()
    if total % batch:
        raise ArError(Status.AR_INVALID_ARGUMENT, "tensor size is not a multiple of batch")
    if stream is None:
        stream = torch.cuda.current_stream(t0.device)
    call = make_call(P, total // batch, rev[dname], op, algo, knob, exec, batch, groups,
                     workspace=workspace, workspace_bytes=(workspace.numel() * workspace.element_size()
                                                           if workspace is not None else 0),
                     collective=collective, steps=steps)
    ar_allreduce_ex(tensors, call, stream)


def reduce_scatter(tensors, algo="ring", op="sum", exec="fused", batch=1, stream=None, workspace=None):
    """In place: tensor q ends with the reduced part q (the ceil split into P parts)."""
    allreduce(tensors, algo, op, 0, exec, batch, None, stream, workspace, "reduce_scatter")


def all_gather(tensors, algo="ring", exec="fused", batch=1, stream=None, workspace=None):
    """In place: tensor q contributes part q; every tensor ends with all parts."""
    allreduce(tensors, algo, "sum", 0, exec, batch, None, stream, workspace, "all_gather")
