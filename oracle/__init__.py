"""CPU oracle of the MoE layer -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import anything from this package.  It shares no code with the
HIP library and never imports it.
"""
from . import moe_oracle, mx, tie_clearance  # noqa: F401
