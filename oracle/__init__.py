"""fp64 CPU oracle for the GQA attention forward/backward.

TEST INFRASTRUCTURE: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import, call or execute anything in
this package.  The HIP library never uses it; see ``oracle.attention`` for the
definitions and their sources.  Every function here is pinned by CPU tests
(finite differences, a library SDPA reduction, invariants, closed forms).
"""
from .attention import (  # noqa: F401
    backward,
    forward,
    forward_backward,
    key_rows,
    query_rows,
    visible,
)
