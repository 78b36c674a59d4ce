"""Plain, slow CPU oracle for the GenRank ranking forward/backward (test infrastructure).

Only the tests, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline leg use this
package.  It shares no code with the HIP library and imports nothing from it.
"""
from .genrank_oracle import *  # noqa: F401,F403
from .genrank_oracle import __all__  # noqa: F401
