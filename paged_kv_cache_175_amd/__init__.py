"""Paged KV-cache attention for MI355X (gfx950).

Hand-written HIP kernels behind a C ABI (``include/pa.h``); this package is
the thin Python binding over it (:mod:`.ops`), the host-side block manager
(:mod:`.pool`) and the seeded synthetic workloads (:mod:`.workloads`).
Importing the package loads nothing; the shared library is loaded on the
first call into :mod:`.ops`, and a missing library is an error.
"""

__all__ = ["ops", "pool", "workloads"]
