"""MI355X-native paged-attention decode.

The compute path is the C-ABI library ``libpa.so`` (hand-written HIP for
gfx950, built in-tree from ``csrc/``); :mod:`.lib` is the thin ctypes binding
with the same entry-point names.  Host helpers: :mod:`.workloads` (seeded
synthetic inputs), :mod:`.block_manager` (refcounts and copy-on-write) and
:mod:`.sizing` (pool arithmetic).
"""
__all__ = ["lib", "workloads", "block_manager", "sizing"]
