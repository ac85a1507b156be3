"""CPU oracle for conditional draft-tree construction -- TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import this package.  It shares no code with the HIP library.
"""
from .dtree_oracle import *  # noqa: F401,F403
from .dtree_oracle import build_round  # noqa: F401
