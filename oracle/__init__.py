"""CPU oracle for the PBD window step — TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of
``bench.py`` may import this package.  The library and its Python binding never
do: the GPU path has no CPU fallback.
"""
from .pbd_oracle import *  # noqa: F401,F403
