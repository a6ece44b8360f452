"""CPU oracle for the AutoRound per-Linear tuning loop.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the HIP library or its
binding. It shares no code with them.
"""
from .autoround_ref import *  # noqa: F401,F403
from .autoround_ref import _pack_axis0, _unpack_axis0  # noqa: F401
