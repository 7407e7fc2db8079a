"""CPU oracle for the cache-guided selective FFN (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The HIP product path never calls it.
"""
from .cgs_oracle import *  # noqa: F401,F403
