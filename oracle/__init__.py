"""CPU oracle for the LOCKS decode path (test infrastructure).

Plain, slow, float64 numpy code written from the LOCKS pages.  Only the tests,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it; the library and its Python binding never do, and the oracle never
imports them.
"""

from .locks_oracle import *  # noqa: F401,F403
