"""CPU oracle for DSA decode-time candidate selection (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  It shares no code with the library.
"""
from .dsa_oracle import *  # noqa: F401,F403
