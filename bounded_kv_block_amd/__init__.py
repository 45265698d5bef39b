"""Bounded-KV block attention on MI355X (gfx950).

``bounded_kv_block_amd.bkv`` is the thin ctypes binding over the C-ABI library
``libbkv.so`` (HIP kernels + host state machine); ``synth`` draws the seeded
synthetic workloads.  Importing this package loads nothing: the library is
opened on first use of the binding and a missing build is an error.
"""
__all__ = ["bkv", "synth"]
