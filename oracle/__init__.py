"""CPU oracle for the routed int4 mixture-of-experts layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The library itself never does, and shares no
code with it.
"""
from .moe_oracle import *  # noqa: F401,F403
