"""Paged decode attention for MI355X (gfx950): slot-mapped KV write, block copy for
copy-on-write, block-table gather and decode-step attention over a shared pool of fixed-size KV
blocks.

The compute path is the C-ABI library ``libpagedattn.so`` (hand-written HIP kernels, declared in
``include/pa.h``). ``paged_kv_cache_318_amd.lib`` is a thin ctypes binding with the same entry
point names; ``paged_kv_cache_318_amd.blocks`` is the host-side block manager that builds block
tables, slots and copy-on-write pairs. Importing this package loads nothing; the library is
opened on first use and a missing library raises an error (there is no fallback path).
"""

__all__ = ["blocks", "lib"]
