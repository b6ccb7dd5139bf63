"""MI355X-native paged-attention decode.

The compute path is the C-ABI library ``libpa.so`` (hand-written HIP for
gfx950, built in-tree from ``csrc/``); :mod:`.lib` is the thin ctypes binding
with the same entry-point names, including the native host block pool
(reference counts, copy-on-write, prefix caching).  Host helpers:
:mod:`.workloads` (seeded synthetic inputs) and :mod:`.sizing` (pool
arithmetic).
"""
__all__ = ["lib", "workloads", "sizing"]
