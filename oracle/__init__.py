"""Plain CPU oracle for the CSA2 sparse-attention hot path.

TEST INFRASTRUCTURE ONLY: the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this package; the product library
never does, and this package never imports the product library.

The arithmetic lives in ``csa2_oracle.c`` (plain C, built with gcc); this module
compiles it and wraps it with numpy.  Parity of every function is pinned by the
``-m "not gpu"`` tests in ``tests/test_oracle_*.py``.  The attention sink is a reading
(the pages only mention that one exists): one more key of value zero, and that arithmetic
is pinned against torch SDPA with an appended zero row.  Parity unpinned: whether V keeps
the RoPE dimensions of the shared latent (the pages do not say; V = K here).
"""
from .oracle import *  # noqa: F401,F403
