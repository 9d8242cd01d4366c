"""CSA2 compressed sparse attention (FP4 indexer) for MI355X / gfx950.

The hot path lives in the HIP library ``libcsa2.so`` (C ABI, ``include/csa2.h``);
``binding`` marshals torch tensors into its entry points.  Importing this package
loads nothing: the library is opened on first use, and a missing library is an
error (there is no other implementation).
"""
__all__ = ["binding", "synth"]
