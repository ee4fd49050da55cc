"""Plain CPU oracle for the paged-KV decode path (fp64 NumPy).

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the product path.
"""
from .pa_oracle import *  # noqa: F401,F403
