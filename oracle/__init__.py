"""CPU oracle for the Dustin sparse-verification step.

TEST INFRASTRUCTURE ONLY: imported by tests, ``__graft_entry__.smoke()`` and
the ``cpu_baseline`` leg of ``bench.py``; never by the product path.
"""
from .dustin import *  # noqa: F401,F403
from .dustin import __all__  # noqa: F401
