"""pagedkv for MI355X: paged KV-cache decode attention, cache writes and a host
block allocator, behind the C ABI of libpagedkv.so (include/pagedkv.h).

The Python layer only marshals arguments; every step of the hot path runs in
the library's hand-written HIP kernels for gfx950.  Device ops live in
``paged_kv_cache_397_amd.ops`` (imports torch); the allocator needs only numpy.
"""

from ._native import PagedKVError, LIB_PATH  # noqa: F401
from .allocator import BlockAllocator  # noqa: F401

__all__ = ["PagedKVError", "BlockAllocator", "LIB_PATH"]
