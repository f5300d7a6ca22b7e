"""fp64 CPU oracle for jagged attention and its tile planner.

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``.  Nothing in the HIP library or
its Python binding imports, links or runs anything in this package.
"""
from . import attention, plan  # noqa: F401
