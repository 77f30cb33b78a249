"""CPU oracle for the AWQ per-layer search — TEST INFRASTRUCTURE.

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline
leg may import anything from this package. The product path (the HIP library
and its Python binding) never imports, links or runs it, and the two share no
code: the oracle is written from the AWQ pages alone.

Every function is pinned by CPU tests in ``tests/test_oracle_pins.py``
(brute force on tiny layers, closed forms, invariants, the storage size the
roadmap page prints). No function here is "parity unpinned".
"""
from .awq_oracle import *  # noqa: F401,F403
from . import awq_oracle  # noqa: F401
