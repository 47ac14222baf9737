"""libmoe: routed int4 mixture-of-experts layer for MI355X (gfx950).

The compute path is the HIP library ``libmoe.so`` (sources in ``csrc/``, C ABI
in ``include/libmoe.h``); ``api`` is its thin ctypes binding with the same
function names.
"""
from . import api  # noqa: F401
