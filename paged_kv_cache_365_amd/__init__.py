"""MI355X-native (gfx950) single-token decode attention over a paged KV cache.

The compute path is the HIP library ``libpa.so`` (C ABI, ``include/pa.h``);
``paged_kv_cache_365_amd.pa`` is its thin ctypes binding.  Importing this package
loads nothing; the binding loads the library on first use and raises if it is
missing.
"""
__all__ = ["pa", "workloads"]
