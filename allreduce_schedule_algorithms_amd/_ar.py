"""ctypes binding of libar_mi355x.so: the C ABI of include/ar.h, same names.

This module only marshals arguments; every step of an Allreduce runs in the
library's HIP kernels. Importing it loads the library and fails loudly when it
is missing (build it with ``python allreduce_schedule_algorithms_amd/build_lib.py``).
"""
from __future__ import annotations

import ctypes as C
import enum
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# AR_LIBRARY may name another build of the same library (for example one built
# with different compiler options); the default is the in-tree build.
LIB_PATH = os.environ.get("AR_LIBRARY") or os.path.join(_HERE, "libar_mi355x.so")

AR_MAX_RANKS = 256


class Status(enum.IntEnum):
    AR_OK = 0
    AR_INVALID_ARGUMENT = 1
    AR_UNSUPPORTED = 2
    AR_WORKSPACE_TOO_SMALL = 3
    AR_HIP_ERROR = 4
    AR_INTERNAL = 5


class Dtype(enum.IntEnum):
    AR_INT32 = 0
    AR_FP32 = 1
    AR_BF16 = 2


class Op(enum.IntEnum):
    AR_SUM = 0
    AR_MAX = 1
    AR_AVG = 2


class Collective(enum.IntEnum):
    AR_ALLREDUCE = 0
    AR_REDUCE_SCATTER = 1
    AR_ALL_GATHER = 2


class Algo(enum.IntEnum):
    AR_DIRECT = 0
    AR_RING = 1
    AR_RH_RD = 2
    AR_RD = 3
    AR_BINOMIAL = 4
    AR_GENERALIZED = 5
    AR_GENERALIZED_XOR = 6
    AR_AHC = 7
    AR_CHAIN = 8
    AR_AUTO = -1


AR_KNOB_AUTO = -1


class CostForm(enum.IntEnum):
    AR_COST_BUSIEST_RANK = 0
    AR_COST_ALL_RANKS = 1


class Kernel(enum.IntEnum):
    AR_KERNEL_NONE = 0
    AR_KERNEL_DIRECT = 1
    AR_KERNEL_LITERAL = 2
    AR_KERNEL_REPLAY = 3
    AR_KERNEL_STAGED = 4
    AR_KERNEL_STRIDED = 5
    AR_KERNEL_FIXED_CHAIN = 6
    AR_KERNEL_FIXED_BALANCED = 7
    AR_KERNEL_FIXED_STACK = 8
    AR_KERNEL_MULTI = 9
    AR_KERNEL_ROWS = 10
    AR_KERNEL_ROWS_VEC = 11
    AR_KERNEL_DAG = 12
    AR_KERNEL_JIT = 13


class Exec(enum.IntEnum):
    AR_EXEC_FUSED = 0
    AR_EXEC_LITERAL = 1
    AR_EXEC_REPLAY = 2
    AR_EXEC_DAG = 3


DTYPES = {"int32": Dtype.AR_INT32, "fp32": Dtype.AR_FP32, "bf16": Dtype.AR_BF16}
OPS = {"sum": Op.AR_SUM, "max": Op.AR_MAX, "avg": Op.AR_AVG}
COLLECTIVES = {"allreduce": Collective.AR_ALLREDUCE, "reduce_scatter": Collective.AR_REDUCE_SCATTER,
               "all_gather": Collective.AR_ALL_GATHER}
ALGOS = {"direct": Algo.AR_DIRECT, "ring": Algo.AR_RING, "rh_rd": Algo.AR_RH_RD, "rd": Algo.AR_RD,
         "binomial": Algo.AR_BINOMIAL, "generalized": Algo.AR_GENERALIZED,
         "generalized_xor": Algo.AR_GENERALIZED_XOR, "ahc": Algo.AR_AHC, "chain": Algo.AR_CHAIN,
         "auto": Algo.AR_AUTO}
ALGO_NAMES = {int(v): k for k, v in ALGOS.items()}
COST_FORMS = {"busiest": CostForm.AR_COST_BUSIEST_RANK, "all_ranks": CostForm.AR_COST_ALL_RANKS}
EXECS = {"fused": Exec.AR_EXEC_FUSED, "literal": Exec.AR_EXEC_LITERAL, "replay": Exec.AR_EXEC_REPLAY,
         "dag": Exec.AR_EXEC_DAG}


class ar_call(C.Structure):
    _fields_ = [("P", C.c_int32), ("dtype", C.c_int32), ("op", C.c_int32), ("algo", C.c_int32),
                ("knob", C.c_int32), ("exec", C.c_int32), ("n", C.c_int64), ("batch", C.c_int64),
                ("ngroups", C.c_int32), ("groups", C.POINTER(C.c_int32)),
                ("workspace", C.c_void_p), ("workspace_bytes", C.c_size_t),
                ("start_event", C.c_void_p), ("stop_event", C.c_void_p), ("collective", C.c_int32),
                ("steps", C.c_int32)]


class ar_oprec(C.Structure):
    _fields_ = [("step", C.c_int32), ("kind", C.c_int32), ("src_rank", C.c_int32), ("src_slot", C.c_int32),
                ("dst_rank", C.c_int32), ("dst_slot", C.c_int32), ("own_slot", C.c_int32),
                ("pair", C.c_int32), ("offset", C.c_int64), ("length", C.c_int64)]


class ar_schedule_info(C.Structure):
    _fields_ = [("steps", C.c_int32), ("slots", C.c_int32), ("atoms", C.c_int32), ("single_port", C.c_int32),
                ("ops", C.c_int64), ("finalize_ops", C.c_int64), ("fused_ok", C.c_int32),
                ("ranges", C.c_int32), ("max_trees", C.c_int32), ("max_need", C.c_int32),
                ("max_leaves", C.c_int32), ("program_words", C.c_int32)]


class ar_cost(C.Structure):
    _fields_ = [("steps", C.c_int32), ("sent_busiest", C.c_int64), ("recv_busiest", C.c_int64),
                ("reduced_busiest", C.c_int64), ("sent_total", C.c_int64), ("reduced_total", C.c_int64),
                ("max_rank_sent", C.c_int64), ("max_rank_reduced", C.c_int64),
                ("predicted_seconds", C.c_double), ("closed_form_seconds", C.c_double),
                ("literal_hbm_bytes", C.c_double), ("fused_hbm_bytes", C.c_double),
                ("essential_bytes", C.c_double)]


class ar_cache_stats(C.Structure):
    _fields_ = [("live_plans", C.c_int64), ("retired_plans", C.c_int64), ("workspaces", C.c_int64),
                ("retired_workspaces", C.c_int64), ("plan_device_bytes", C.c_int64),
                ("workspace_device_bytes", C.c_int64)]


class ar_cost_model(C.Structure):
    _fields_ = [("alpha", C.c_double), ("beta", C.c_double), ("gamma", C.c_double), ("form", C.c_int32),
                ("reserved", C.c_int32)]


# exported symbol -> (restype, argtypes)
SIGNATURES = {
    "ar_allreduce": (C.c_int, [C.POINTER(C.c_void_p), C.c_int32, C.c_int64, C.c_int32, C.c_int32, C.c_int32,
                               C.c_int32, C.c_void_p]),
    "ar_allreduce_ex": (C.c_int, [C.POINTER(C.c_void_p), C.POINTER(ar_call), C.c_void_p]),
    "ar_allreduce_noalloc": (C.c_int, [C.POINTER(C.c_void_p), C.POINTER(ar_call), C.c_void_p]),
    "ar_reduce_scatter": (C.c_int, [C.POINTER(C.c_void_p), C.c_int32, C.c_int64, C.c_int32, C.c_int32,
                                    C.c_int32, C.c_void_p]),
    "ar_all_gather": (C.c_int, [C.POINTER(C.c_void_p), C.c_int32, C.c_int64, C.c_int32, C.c_int32, C.c_void_p]),
    "ar_workspace_bytes": (C.c_int, [C.POINTER(ar_call), C.POINTER(C.c_size_t)]),
    "ar_set_launch_blocks": (C.c_int, [C.c_int64, C.POINTER(C.c_int64)]),
    "ar_cache_stats_get": (C.c_int, [C.POINTER(ar_cache_stats)]),
    "ar_release_cached": (C.c_int, []),
    "ar_kernel_of": (C.c_int, [C.POINTER(ar_call), C.POINTER(C.c_int32)]),
    "ar_schedule_build": (C.c_int, [C.POINTER(ar_call), C.POINTER(C.c_void_p)]),
    "ar_schedule_info_get": (C.c_int, [C.c_void_p, C.POINTER(ar_schedule_info)]),
    "ar_schedule_export": (C.c_int, [C.c_void_p, C.POINTER(ar_oprec), C.c_size_t, C.POINTER(C.c_size_t)]),
    "ar_schedule_fused_export": (C.c_int, [C.c_void_p, C.POINTER(C.c_int64), C.POINTER(C.c_int64),
                                           C.POINTER(C.c_int32), C.c_size_t, C.POINTER(C.c_int32), C.c_size_t,
                                           C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "ar_schedule_dag_export": (C.c_int, [C.c_void_p, C.POINTER(C.c_int32), C.POINTER(C.c_int32), C.c_size_t,
                                         C.POINTER(C.c_uint8), C.c_size_t, C.POINTER(C.c_int32), C.c_size_t,
                                         C.POINTER(C.c_size_t), C.POINTER(C.c_size_t), C.POINTER(C.c_size_t)]),
    "ar_schedule_free": (None, [C.c_void_p]),
    "ar_table_check": (C.c_int, [C.c_int32, C.c_int64, C.c_int32, C.POINTER(ar_oprec), C.c_size_t,
                                 C.POINTER(C.c_int32)]),
    "ar_table_check_ex": (C.c_int, [C.POINTER(ar_call), C.POINTER(ar_oprec), C.c_size_t, C.POINTER(C.c_int32)]),
    "ar_cost_report": (C.c_int, [C.c_void_p, C.c_double, C.c_double, C.c_double, C.POINTER(ar_cost)]),
    "ar_cost_steps": (C.c_int, [C.c_void_p, C.POINTER(C.c_int64), C.POINTER(C.c_int64), C.POINTER(C.c_int64)]),
    "ar_set_cost_model": (C.c_int, [C.POINTER(ar_cost_model)]),
    "ar_get_cost_model": (C.c_int, [C.POINTER(ar_cost_model)]),
    "ar_select": (C.c_int, [C.POINTER(ar_call), C.POINTER(C.c_int32), C.POINTER(C.c_int32),
                            C.POINTER(C.c_double)]),
    "ar_status_string": (C.c_char_p, [C.c_int]),
    "ar_last_hip_error": (C.c_int32, []),
    "ar_last_error_message": (C.c_char_p, []),
    "ar_version": (C.c_char_p, []),
}


def _load():
    # Device memory and streams come from PyTorch, which ships its own HIP
    # runtime (libamdhip64.so.7). Loading torch first makes the library's
    # libamdhip64.so.7 dependency resolve to that same runtime, so tensors'
    # pointers and torch streams are valid in the library's calls.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python allreduce_schedule_algorithms_amd/build_lib.py` "
            "(there is no fallback path)")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


lib = _load()


class ArError(RuntimeError):
    def __init__(self, status: int, message: str):
        self.status = Status(status)
        super().__init__(f"{self.status.name}: {message}")


def _check(st: int):
    if st != Status.AR_OK:
        raise ArError(st, lib.ar_last_error_message().decode())


def _ptrs(bufs):
    if isinstance(bufs, C.Array):  # already marshalled (c_void_p * P), e.g. reused across calls
        return bufs
    ptrs = [b if isinstance(b, int) else b.data_ptr() for b in bufs]
    return (C.c_void_p * max(len(ptrs), 1))(*ptrs)


def marshal_ptrs(bufs):
    """The host array of P device pointers an entry point takes, built once: a
    caller that repeats calls on the same buffers passes it instead of a list."""
    return _ptrs(bufs)


def _stream(stream):
    if stream is None:
        return None
    if isinstance(stream, int):
        return C.c_void_p(stream)
    return C.c_void_p(stream.cuda_stream)  # a torch.cuda.Stream


def _enum(table, v):
    return int(table[v]) if isinstance(v, str) else int(v)


def _event(ev):
    if ev is None or isinstance(ev, int):
        return ev
    return ev.cuda_event  # a torch.cuda.Event that has been recorded once (so it exists)


def make_call(P, n, dtype, op="sum", algo="ring", knob=0, exec="fused", batch=1, groups=None,
              workspace=None, workspace_bytes=0, start_event=None, stop_event=None, collective="allreduce",
              steps=0):
    call = ar_call()
    call.collective = _enum(COLLECTIVES, collective)
    call.steps = int(steps)
    call.P, call.n, call.batch = int(P), int(n), int(batch)
    call.dtype, call.op = _enum(DTYPES, dtype), _enum(OPS, op)
    call.algo, call.knob, call.exec = _enum(ALGOS, algo), int(knob), _enum(EXECS, exec)
    if groups:
        arr = (C.c_int32 * len(groups))(*groups)
        call.ngroups, call.groups = len(groups), C.cast(arr, C.POINTER(C.c_int32))
        call._groups_keepalive = arr
    else:
        call.ngroups, call.groups = 0, None
    call.workspace = workspace if isinstance(workspace, (int, type(None))) else workspace.data_ptr()
    call.workspace_bytes = int(workspace_bytes)
    call.start_event, call.stop_event = _event(start_event), _event(stop_event)
    return call


# ---- the C entry points, same names ----
def ar_allreduce(bufs, P, n, dtype, op, algo, knob=0, stream=None):
    _check(lib.ar_allreduce(_ptrs(bufs), int(P), int(n), _enum(DTYPES, dtype), _enum(OPS, op),
                            _enum(ALGOS, algo), int(knob), _stream(stream)))


def ar_reduce_scatter(bufs, P, n, dtype, op, algo, stream=None):
    _check(lib.ar_reduce_scatter(_ptrs(bufs), int(P), int(n), _enum(DTYPES, dtype), _enum(OPS, op),
                                 _enum(ALGOS, algo), _stream(stream)))


def ar_all_gather(bufs, P, n, dtype, algo, stream=None):
    _check(lib.ar_all_gather(_ptrs(bufs), int(P), int(n), _enum(DTYPES, dtype), _enum(ALGOS, algo),
                             _stream(stream)))


def ar_allreduce_ex(bufs, call: ar_call, stream=None):
    _check(lib.ar_allreduce_ex(_ptrs(bufs), C.byref(call), _stream(stream)))


AR_NOALLOC_SCRATCH_BYTES = 64 << 20


def ar_allreduce_noalloc(bufs, call: ar_call, stream=None):
    """Allocation-free variant of ar_allreduce_ex (literal execution, scratch in a static device array)."""
    _check(lib.ar_allreduce_noalloc(_ptrs(bufs), C.byref(call), _stream(stream)))


def ar_workspace_bytes(call: ar_call) -> int:
    out = C.c_size_t(0)
    _check(lib.ar_workspace_bytes(C.byref(call), C.byref(out)))
    return out.value


def ar_kernel_of(call: ar_call) -> Kernel:
    """The kernel family the call runs (host only)."""
    out = C.c_int32(0)
    _check(lib.ar_kernel_of(C.byref(call), C.byref(out)))
    return Kernel(out.value)


def ar_cache_stats_get() -> dict:
    """Plans and workspaces the library holds (live and retired) and their device bytes."""
    out = ar_cache_stats()
    _check(lib.ar_cache_stats_get(C.byref(out)))
    return {name: getattr(out, name) for name, _ in ar_cache_stats._fields_}


def ar_release_cached() -> None:
    """Free every plan, workspace and cached schedule (see include/ar.h for the conditions)."""
    _check(lib.ar_release_cached())


def ar_set_launch_blocks(max_blocks: int) -> int:
    """Set the per-launch workgroup limit; returns the previous one."""
    prev = C.c_int64(0)
    _check(lib.ar_set_launch_blocks(int(max_blocks), C.byref(prev)))
    return prev.value


def ar_schedule_build(call: ar_call) -> "Schedule":
    h = C.c_void_p()
    _check(lib.ar_schedule_build(C.byref(call), C.byref(h)))
    return Schedule(h)


def ar_table_check(P, n, dtype, ops) -> bool:
    """Returns the single-port flag; raises ArError when the table is not a correct Allreduce."""
    arr = (ar_oprec * max(len(ops), 1))(*ops)
    sp = C.c_int32(0)
    _check(lib.ar_table_check(int(P), int(n), _enum(DTYPES, dtype), arr, len(ops), C.byref(sp)))
    return bool(sp.value)


def ar_set_cost_model(alpha=None, beta=None, gamma=None, form="all_ranks"):
    """Set the process-wide model; with no arguments restore the default."""
    if alpha is None and beta is None and gamma is None:
        _check(lib.ar_set_cost_model(None))
        return
    m = ar_cost_model(float(alpha), float(beta), float(gamma), _enum(COST_FORMS, form), 0)
    _check(lib.ar_set_cost_model(C.byref(m)))


def ar_get_cost_model() -> dict:
    m = ar_cost_model()
    _check(lib.ar_get_cost_model(C.byref(m)))
    names = {int(v): k for k, v in COST_FORMS.items()}
    return dict(alpha=m.alpha, beta=m.beta, gamma=m.gamma, form=names[m.form])


def ar_select(call: ar_call):
    """(algorithm name, knob, model seconds) of the schedule the call runs."""
    a, k, t = C.c_int32(0), C.c_int32(0), C.c_double(0)
    _check(lib.ar_select(C.byref(call), C.byref(a), C.byref(k), C.byref(t)))
    return ALGO_NAMES[a.value], k.value, t.value


def ar_table_check_ex(call: ar_call, ops) -> bool:
    """ar_table_check for the call's collective; returns the single-port flag."""
    arr = (ar_oprec * max(len(ops), 1))(*ops)
    sp = C.c_int32(0)
    _check(lib.ar_table_check_ex(C.byref(call), arr, len(ops), C.byref(sp)))
    return bool(sp.value)


def ar_status_string(st) -> str:
    return lib.ar_status_string(int(st)).decode()


def ar_last_hip_error() -> int:
    return int(lib.ar_last_hip_error())


def ar_last_error_message() -> str:
    return lib.ar_last_error_message().decode()


def ar_version() -> str:
    return lib.ar_version().decode()


class Schedule:
    """Owned ar_schedule handle (host-only step table, fused program and cost walk)."""

    def __init__(self, handle: C.c_void_p):
        self._h = handle

    def __del__(self):
        # at interpreter exit the module's globals may already be gone; the
        # process then releases the schedule with everything else
        if getattr(self, "_h", None) and lib is not None:
            lib.ar_schedule_free(self._h)
            self._h = None

    def info(self) -> ar_schedule_info:
        out = ar_schedule_info()
        _check(lib.ar_schedule_info_get(self._h, C.byref(out)))
        return out

    def export(self):
        cnt = C.c_size_t(0)
        _check(lib.ar_schedule_export(self._h, None, 0, C.byref(cnt)))
        arr = (ar_oprec * max(cnt.value, 1))()
        _check(lib.ar_schedule_export(self._h, arr, cnt.value, C.byref(cnt)))
        return list(arr[: cnt.value])

    def fused_export(self):
        nr, nw = C.c_size_t(0), C.c_size_t(0)
        _check(lib.ar_schedule_fused_export(self._h, None, None, None, 0, None, 0, C.byref(nr), C.byref(nw)))
        starts = (C.c_int64 * max(nr.value, 1))()
        lens = (C.c_int64 * max(nr.value, 1))()
        offs = (C.c_int32 * max(nr.value, 1))()
        words = (C.c_int32 * max(nw.value, 1))()
        _check(lib.ar_schedule_fused_export(self._h, starts, lens, offs, nr.value, words, nw.value,
                                            C.byref(nr), C.byref(nw)))
        return list(starts[: nr.value]), list(lens[: nr.value]), list(offs[: nr.value]), list(words[: nw.value])

    def dag_export(self):
        """(shared, offsets per range, maps as a (ranges, P) array or None, program words)."""
        import numpy as np
        sh = C.c_int32(0)
        nr, nm, nw = C.c_size_t(0), C.c_size_t(0), C.c_size_t(0)
        _check(lib.ar_schedule_dag_export(self._h, C.byref(sh), None, 0, None, 0, None, 0, C.byref(nr),
                                          C.byref(nm), C.byref(nw)))
        offs = (C.c_int32 * max(nr.value, 1))()
        maps = (C.c_uint8 * max(nm.value, 1))()
        words = (C.c_int32 * max(nw.value, 1))()
        _check(lib.ar_schedule_dag_export(self._h, C.byref(sh), offs, nr.value, maps, nm.value, words, nw.value,
                                          C.byref(nr), C.byref(nm), C.byref(nw)))
        m = np.frombuffer(bytes(maps[: nm.value]), dtype=np.uint8).reshape(nr.value, -1) if nm.value else None
        return bool(sh.value), list(offs[: nr.value]), m, list(words[: nw.value])

    def cost(self, alpha=0.0, beta=0.0, gamma=0.0) -> ar_cost:
        out = ar_cost()
        _check(lib.ar_cost_report(self._h, float(alpha), float(beta), float(gamma), C.byref(out)))
        return out

    def cost_steps(self, P):
        inf = self.info()
        n = max(inf.steps * P, 1)
        s, r, d = (C.c_int64 * n)(), (C.c_int64 * n)(), (C.c_int64 * n)()
        _check(lib.ar_cost_steps(self._h, s, r, d))
        import numpy as np
        shape = (inf.steps, P)
        return (np.array(s[: inf.steps * P]).reshape(shape), np.array(r[: inf.steps * P]).reshape(shape),
                np.array(d[: inf.steps * P]).reshape(shape))
