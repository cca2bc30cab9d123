"""CPU oracle for the routed-expert MoE forward layer (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import this package; the HIP library and its binding never do.
"""
from .moe_oracle import *  # noqa: F401,F403
