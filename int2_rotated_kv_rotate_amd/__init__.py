"""Rotated INT2 KV cache with mixed-precision paged decode attention for MI355X (gfx950).

The compute lives in a HIP shared library (``csrc/``) behind a C ABI (``include/oscar.h``);
``ops`` is a thin ctypes binding over it that only marshals torch tensors into pointers.
Importing this package does not load the library; the first call into ``ops`` does, and
raises if the library has not been built.
"""
__all__ = ["workload", "ops"]
