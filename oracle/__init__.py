"""CPU oracle (test infrastructure only; see ``oracle/rrs_ref.py``).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package.
"""
from .rrs_ref import *  # noqa: F401,F403
from .rrs_ref import QMAX  # noqa: F401
