"""CPU oracle for the Allreduce schedules -- TEST INFRASTRUCTURE ONLY.

Plain, slow, obviously correct NumPy replays of what each schedule on the
pages computes, written from the pages and independent of the HIP library:
it imports nothing from ``allreduce_schedule_algorithms_amd`` and shares no
code, table or helper with it. Only ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py`` may import it; the product path
never does.

Modules
-------
numerics   the reduction algebras (int32 wrap-around sum, fp32 sum, bf16 sum
           with fp32 partials, total-order max, a symbolic tree algebra), the
           fp64 reference and summation error bounds.
net        a P-rank message simulator with snapshot step semantics and
           per-rank traffic counters.
schedules  one replay per schedule: direct, ring, recursive halving +
           doubling, recursive doubling, binomial tree + broadcast, the
           group-theoretic generalized Allreduce (cyclic and XOR groups, knob
           r) and AHC.
cost       the alpha-beta-gamma closed forms and the bandwidth arithmetic the
           pages state in prose.

Parity status: every function here is pinned by a test under ``tests/`` that
does not re-type its formula (brute force, printed counts, structural
equivalences between independently written schedules, symbolic trees, closed
error bounds). The exact fp32/bf16 bits of a schedule are not printed on any
page; they are pinned only through those invariants (see the per-function
notes in ``schedules``).
"""
from . import numerics, net, schedules, cost  # noqa: F401
from .schedules import allreduce, ALGOS  # noqa: F401
