"""CPU oracle for the routed int4 mixture-of-experts layer (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The library itself never does, and shares no
code with it.

``import oracle`` gives the oracle the GPU is checked against: the plain C++17
fp32 implementation (``moe_oracle.cpp``, through ``oracle.cpp``).
``oracle.fp64`` is the float64 numpy form of the same definitions, used to
cross-check it.
"""
from . import fp64  # noqa: F401
from .cpp import *  # noqa: F401,F403
from .cpp import build, lib, set_threads, threads, route32, router_logits2, experts_combine  # noqa: F401
