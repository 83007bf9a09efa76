"""Build libar_mi355x.so (the Allreduce library) and libar_probe.so (memory-traffic
ceiling kernels for measurement) in-tree with hipcc for gfx950.

Usage: python allreduce_schedule_algorithms_amd/build_lib.py   (or __graft_entry__.build())
Run it as a file, not as a package module: importing the package loads the library.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "csrc")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libar_mi355x.so")
PROBE_LIB = os.path.join(HERE, "libar_probe.so")
ROOT = os.path.dirname(HERE)

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", "-I", os.path.join(ROOT, "include")]
# Device code: no packed-fp32 instructions, no FMA contraction, IEEE denormals
# (the replay must reproduce the step list's rounding bit for bit).
DEVICE = [f"--offload-arch={ARCH}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-ffp-contract=off", "-fno-gpu-flush-denormals-to-zero", "-fno-fast-math"]

SOURCES = [
    ("sched.cpp", False),
    ("abi.cpp", False),
    ("jit.cpp", False),
    ("exec.hip", True),
] + [(f"launch_{d}_{o}.hip", True) for d in ("i32", "f32", "bf16") for o in ("sum", "max")] + \
    [(f"launch_{d}_avg.hip", True) for d in ("f32", "bf16")]


def _compile(src: str, device: bool) -> str:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC] + COMMON + (DEVICE + ["-x", "hip"] if device else ["-ffp-contract=off"]) + \
        ["-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"compile failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    return obj


def _link(objs, out: str) -> None:
    tmp = out + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp] + objs
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed: {' '.join(cmd)}\n{r.stdout}\n{r.stderr}")
    os.replace(tmp, out)


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    srcs = SOURCES + [("probe.hip", True)]
    with cf.ThreadPoolExecutor(max_workers=min(len(srcs), os.cpu_count() or 4, 16)) as ex:
        objs = list(ex.map(lambda s: _compile(*s), srcs))
    _link(objs[:-1], LIB)
    _link(objs[-1:], PROBE_LIB)
    if verbose:
        print(f"built {LIB} and {PROBE_LIB}")
    return LIB


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
