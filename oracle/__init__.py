"""CPU oracle for the paged KV-cache hot path -- TEST INFRASTRUCTURE ONLY.

This package is a plain, slow, obviously-correct fp64 restatement of what the
paged KV-cache path computes.  It exists to check the HIP path, and it is only
ever imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The product package never imports it,
and it never imports the product package: the two share no code.  The only
thing both sides consume is the seeded input generator, which holds none of
the method's arithmetic.

Sources (the pages this restates, cited by title and section):

* "PagedAttention in mistral.rs" (mistral.rs docs): KV cache split into
  fixed-size token blocks (default 32) addressed per sequence; the pool is
  sized from a memory budget and a block size; optional F8E4M3 cache type.
* "Optimization plans" (mistral.rs discussion 46), the "Update" post: the
  cache slot writer ``reshape_and_cache`` runs before paged attention.
* "libmir-metal 0.2.0, src/native/trace/kv.rs", ``fn build``: head-major
  pages; sliding layers keep a bounded ring; a quantised cache holds packed
  INT8 pages with per-token/head FP32 scales, dequantised inside attention.
* "Rolling buffer cache" (llama.cpp discussion 3581), opening post: a cache of
  fixed size W holds timestep i at slot i mod W; KerfuffleV2's reply states the
  sliding-window span of a token.

Modules:

* :mod:`oracle.e4m3`     -- OCP E4M3 ("FN") table, brute-force RNE encoder.
* :mod:`oracle.int8`     -- symmetric per-(token, head) int8 codes, fp32 scales.
* :mod:`oracle.cache`    -- slot arithmetic and the cache writer.
* :mod:`oracle.attention` -- paged decode, rolling-buffer decode, chunked
  prefill, split-context merge.
* :mod:`oracle.pool`     -- pool sizing arithmetic and ring-slot rule.

Every function here has at least one pin in ``tests/test_oracle_*.py`` that
ties it to something other than itself (closed forms, a library routine,
invariants, brute force).  No function is "parity unpinned".
"""

from . import e4m3, cache, attention, pool  # noqa: F401
