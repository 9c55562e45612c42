"""CPU fp64 oracle for the DSA sparse decode step (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package; the product path never does.
"""
from .dsa_oracle import *  # noqa: F401,F403
from . import dsa_oracle  # noqa: F401
