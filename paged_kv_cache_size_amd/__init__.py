"""Paged KV-cache write and paged decode attention for AMD MI355X (gfx950).

The compute lives in the HIP library ``libpa.so`` (C ABI, ``include/pa.h``);
this package is its thin Python binding plus the seeded workload builders.
"""
