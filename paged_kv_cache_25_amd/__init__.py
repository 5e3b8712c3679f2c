"""Decode-step attention over a paged KV cache, for MI355X (gfx950).

The work is done by three HIP kernels behind the C ABI in ``include/pkv.h``
(``libpkv.so``, built in-tree from ``csrc/``).  ``paged_kv_cache_25_amd.ops``
is a thin ctypes binding over it that takes torch tensors for device memory
and the current HIP stream; it raises if the library is missing.  Importing
this package loads nothing.
"""

__all__ = ["ops", "traffic"]
