"""CPU oracle for the KVpop fixed-budget KV-cache hot path (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s ``cpu_baseline``
leg may import this package; the HIP library never does, and this package never
imports the HIP library.
"""
from .kvpop_oracle import *  # noqa: F401,F403
from .kvpop_oracle import INT32_MAX  # noqa: F401
