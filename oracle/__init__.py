"""fp64 CPU oracle of the TurboQuant KV-cache hot path -- TEST INFRASTRUCTURE.

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import
this package.  It shares no code with the HIP library or its binding.
"""
from .turboquant import *  # noqa: F401,F403
