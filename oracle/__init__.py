"""Float64 CPU oracle for split-KV partial decode attention.

TEST INFRASTRUCTURE ONLY. Nothing in the library imports this package; only the
test suite, the smoke check and the CPU-baseline leg of the benchmark may use it.
It shares no code with the HIP path (no kernels, headers, helpers or tables);
both sides receive the same seeded inputs from the separate ``workloads`` module.

Contents
--------
``attention``  plain definitions: gather through the page table, full softmax
               attention, partial attention over a KV subset, LSE merge.
``planner``    the critical-wave split planner of LiquidCP section 5.2, written as
               a slow, direct event simulation plus greedy search.

Every function cites the passage of the pages it follows. Parity status of each
function (what pins it) is stated in its docstring; all functions here are
pinned by tests under ``tests/test_oracle_*.py`` and ``tests/test_planner_ref.py``.
"""
from . import attention, planner  # noqa: F401
