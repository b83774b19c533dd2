"""Paged K/V cache decode for AMD Instinct MI355X (gfx950).

* ``ops`` -- torch binding of the C ABI (include/pa.h): ``store_kv``,
  ``copy_pages``, ``decode`` (with sinks), ``prefill``, ``update_tables``.  The HIP library is loaded on first call and a
  missing library is an error, never a fallback.
* ``alloc`` -- the host block allocator that produces block tables, slot
  tables, new-row slots, copy-on-write copy lists and per-step table updates.
* ``memory`` -- capacity, waste and fragmentation report over the allocator.
"""
from . import alloc, memory, ops
from .alloc import OutOfPages, PagedKVCache

__all__ = ["alloc", "memory", "ops", "OutOfPages", "PagedKVCache"]
