"""CPU oracle for the MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never imports, calls or links it, and it shares no code
with that path.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
