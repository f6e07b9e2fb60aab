"""CPU fp64 oracle of the MoE-layer forward.

TEST INFRASTRUCTURE ONLY.  Only tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py may import this package.  The HIP product path
never calls it and shares no code with it.
"""
from .moe_oracle import *  # noqa: F401,F403
