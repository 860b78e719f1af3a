"""Paged decode attention for AMD MI355X (gfx950).

The compute path lives in ``libpa.so`` (HIP kernels behind a C ABI, declared in
``include/pa.h``).  ``paged_kv_cache_05_amd.ops`` is the thin ctypes binding over it;
``block_manager`` is the host-side block engine that builds block tables, slot
mappings and copy-on-write pairs; ``workloads`` draws seeded synthetic inputs.

Importing this package loads nothing; ``ops`` loads the library on first use and
raises if it is missing.
"""

__all__ = ["ops", "block_manager", "workloads"]
