"""CPU oracle for the SOCKET decode path -- TEST INFRASTRUCTURE ONLY.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg may import this package.  The product path never does.
"""
from . import socket_oracle, brute  # noqa: F401
