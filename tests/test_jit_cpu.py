"""The compiled register DAG on the host: which calls take it, what AR_TRACE
says about it, and the kernels that run instead with AR_JIT=0 (no GPU needed:
hipRTC compiles for gfx950 without one)."""
import os
import subprocess
import sys

import allreduce_schedule_algorithms_amd as A

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _choices(env_extra):
    code = ("import allreduce_schedule_algorithms_amd as A\n"
            "for P, n, r in ((7, 1 << 24, 3), (7, 1 << 24, 1), (12, 4099, 2), (13, 1000, 4)):\n"
            "    st = 4 if P == 13 else 0\n"
            "    print(int(A.ar_kernel_of(A.make_call(P, n, 'fp32', 'sum', 'generalized', r, steps=st))))\n")
    env = dict(os.environ, **env_extra)
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True, timeout=300)
    assert r.returncode == 0, r.stderr
    return [int(x) for x in r.stdout.split()], r.stderr


def test_jit_choice_trace_and_off_switch():
    K = A.Kernel
    on, err = _choices({"AR_TRACE": "1"})
    assert on == [K.AR_KERNEL_JIT] * 4
    lines = [ln for ln in err.splitlines() if ln.startswith("ar: plan ")]
    assert len(lines) == 4 and all("kernel ar_jit" in ln and "compiled register DAG" in ln for ln in lines), err
    off, _ = _choices({"AR_JIT": "0"})
    assert off == [K.AR_KERNEL_MULTI, K.AR_KERNEL_MULTI, K.AR_KERNEL_DAG, K.AR_KERNEL_DAG]


def test_jit_takes_no_workspace_and_keeps_batches_of_short_ranges_elsewhere():
    K = A.Kernel
    call = A.make_call(7, 1 << 24, "bf16", "max", "generalized", 2)
    assert A.ar_kernel_of(call) == K.AR_KERNEL_JIT
    assert A.ar_workspace_bytes(call) == 0
    # short ranges of a batch: strided work, not the compiled kernel
    assert A.ar_kernel_of(A.make_call(24, 106, "fp32", "sum", "generalized", 1, batch=10_000)) == K.AR_KERNEL_STRIDED
    # 17 ranges (one per rank), more than the compiled form's 16: the DAG replay
    assert A.ar_kernel_of(A.make_call(17, 5000, "fp32", "sum", "generalized", 2)) == K.AR_KERNEL_DAG


def test_table_form_choice_trace_and_off_switch():
    # one range of one tree over more than 32 ranks: the tree shape compiled
    # with a rank table; many ranges (the ring, the generalized algorithm over
    # Z_P) keep the program-driven replay; latency-bound calls the DAG replay
    code = ("import allreduce_schedule_algorithms_amd as A\n"
            "for P, n, algo, k, dt in ((33, 5000, 'rh_rd', 0, 'fp32'), (192, 1 << 20, 'binomial', 0, 'bf16'),\n"
            "                          (127, 9000, 'chain', 1, 'int32'), (192, 1 << 20, 'ring', 0, 'bf16'),\n"
            "                          (100, 9000, 'generalized', 0, 'fp32'), (200, 4096, 'rh_rd', 0, 'fp32')):\n"
            "    print(int(A.ar_kernel_of(A.make_call(P, n, dt, 'sum', algo, k))))\n")
    K = A.Kernel

    def run(extra):
        env = dict(os.environ, **extra)
        r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, env=env, capture_output=True, text=True,
                           timeout=300)
        assert r.returncode == 0, r.stderr
        return [int(x) for x in r.stdout.split()], r.stderr

    on, err = run({"AR_TRACE": "1"})
    assert on == [K.AR_KERNEL_JIT] * 3 + [K.AR_KERNEL_REPLAY, K.AR_KERNEL_REPLAY, K.AR_KERNEL_DAG], on
    table = [ln for ln in err.splitlines() if "tree shape with a rank table" in ln]
    assert len(table) == 3 and all("kernel ar_jit" in ln for ln in table), err
    off, _ = run({"AR_JIT": "0"})
    assert off == [K.AR_KERNEL_REPLAY] * 5 + [K.AR_KERNEL_DAG], off
