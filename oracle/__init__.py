"""The fp64 CPU oracle for exact attention (TEST INFRASTRUCTURE).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg
may import it.  It shares no code with the HIP path.
"""
from .attention import *  # noqa: F401,F403
from .attention import __all__  # noqa: F401
