"""Plain float64 CPU oracle for TurboQuant (test infrastructure only).

Only `tests/`, `__graft_entry__.smoke()` and the `cpu_baseline` leg of
`bench.py` may import or call anything in this package. The HIP product path
never imports it, and it imports nothing from the product path.
"""
from .tq_oracle import *  # noqa: F401,F403
