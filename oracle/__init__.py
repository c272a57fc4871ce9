"""Oracle for block-sparse masked attention: TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import it. It shares no code with the HIP path.
"""
from . import brute, oracle  # noqa: F401
