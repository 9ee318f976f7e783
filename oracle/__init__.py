"""CPU oracle for the weight-shared looped transformer — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The GPU library never calls it, links it or
reads anything it produced; the two share no code.  Inputs come from ``synth``.

Everything is plain numpy in float64 unless a ``dt`` argument says otherwise;
matrix products use numpy's matmul as a library primitive.  Each function names
the passage of the pages it follows.  Parity status of each function is listed in
``oracle.model.__doc__``.
"""
from .model import *  # noqa: F401,F403
