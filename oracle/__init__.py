"""Plain fp64 CPU oracle for paged decode attention and its KV-cache moves.

TEST INFRASTRUCTURE, NOT PRODUCT CODE. Only the test suite, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import anything from this package. It shares no code with
the HIP library (``paged_kv_cache_318_amd``) and imports nothing from it; the two meet only in the
seeded host arrays that ``workloads`` draws.

Every function in ``oracle.reference`` is pinned by a ``-m "not gpu"`` test to something other
than itself (the printed worked example, closed forms, a textbook/library routine, brute force).
No function here is "parity unpinned".
"""

from .reference import *  # noqa: F401,F403
