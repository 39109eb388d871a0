"""fp64 CPU oracle of the DSpark sampling step.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``; never by the library.
"""
from .dspark_oracle import *  # noqa: F401,F403
from .dspark_oracle import __all__  # noqa: F401
