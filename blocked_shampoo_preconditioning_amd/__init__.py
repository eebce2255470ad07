"""Blocked Shampoo optimizer step for AMD Instinct MI355X (gfx950).

The compute runs in a HIP shared library (``libshampoo_mi355x.so``) behind a
C ABI declared in ``include/shampoo.h``; ``shampoo`` holds the thin ctypes
binding. Importing this package loads nothing; the library is loaded on first
use and a missing library is an error, never a fallback.
"""

__all__ = ["configs", "synth"]
