"""ctypes binding of libar_probe.so (include/ar_probe.h): memory-traffic ceilings
for the Allreduce's access pattern, used by the benchmark. Measurement only; the
Allreduce path never loads it."""
from __future__ import annotations

import ctypes as C
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libar_probe.so")

AR_PROBE_STREAMS = 0
AR_PROBE_COPY = 1
AR_PROBE_FOLD = 2

SIGNATURES = {
    "ar_probe_stream": (C.c_int32, [C.POINTER(C.c_void_p), C.c_int32, C.c_int64, C.c_int32, C.c_int32,
                                    C.c_void_p, C.c_void_p, C.c_void_p]),
    "ar_probe_last_hip_error": (C.c_int32, []),
}


def _load():
    import torch  # noqa: F401  (the HIP runtime that owns the tensors and streams)
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python allreduce_schedule_algorithms_amd/build_lib.py`")
    lib = C.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(lib, name)
        f.restype = res
        f.argtypes = args
    return lib


_lib = None


def lib():
    global _lib
    if _lib is None:
        _lib = _load()
    return _lib


def ar_probe_stream(ptrs, nbytes: int, kind: int, vectors_per_thread: int, stream=None, start_event=None,
                    stop_event=None) -> None:
    arr = (C.c_void_p * len(ptrs))(*ptrs)
    st = None if stream is None else C.c_void_p(stream if isinstance(stream, int) else stream.cuda_stream)
    rc = lib().ar_probe_stream(arr, len(ptrs), int(nbytes), int(kind), int(vectors_per_thread), st,
                               start_event, stop_event)
    if rc:
        raise RuntimeError(f"ar_probe_stream failed ({rc}, HIP error {lib().ar_probe_last_hip_error()})")
