"""Plain fp64 CPU oracle for paged MLA decode / causal multi-token verify over
a round-robin context-sharded KV cache.

TEST INFRASTRUCTURE ONLY. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package. It shares no code
with the HIP library in ``mla_paged_decode_verify_amd`` and never imports it.

Every function in ``oracle.mla`` is pinned by a ``-m "not gpu"`` test in
``tests/test_oracle_pins.py`` against something other than itself (closed
forms, hand-worked examples, brute force, invariants, library routines).
"""

from .mla import *  # noqa: F401,F403
