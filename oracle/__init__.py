"""Float64 CPU oracle for OAL causal attention (test infrastructure only).

Only the test suite, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""
from .oal_oracle import *  # noqa: F401,F403
