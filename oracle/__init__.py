"""Plain CPU oracle for the CSA2 sparse-attention hot path.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product library
never does, and this package never imports the product library.

The arithmetic lives in ``csa2_oracle.c`` (plain C, built with gcc); this module
compiles it and wraps it with numpy.  Parity of every function is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle_*.py``; the one unpinned behaviour
(attention sink semantics) is marked "parity unpinned" where it appears.
"""
from .oracle import *  # noqa: F401,F403
