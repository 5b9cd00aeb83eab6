"""CPU oracle of the MoE layer forward (test infrastructure only).

Imported by ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline``
leg of ``bench.py``; never by the product path.
"""
from . import moe  # noqa: F401
