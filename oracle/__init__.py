"""CPU oracle (test infrastructure only).

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of ``bench.py``
may import or run anything under ``oracle/``.  The oracle shares no code with the HIP
library; both read the same seeded inputs from ``synth``.
"""
from . import dflash_oracle  # noqa: F401
from .dflash_oracle import *  # noqa: F401,F403
