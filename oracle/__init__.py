"""CPU oracle for paged KV-cache attention — TEST INFRASTRUCTURE ONLY.

A plain, slow fp64 NumPy statement of what the paged-attention hot path computes,
used to check the HIP library.  Only the test suite, the package smoke check and
the benchmark's CPU-baseline leg may import it; the library and its Python
binding never do, and this package imports nothing from them.

Contents
  paged_attention  scatter of new K/V rows into pool slots, whole-block copies
                   for copy-on-write, block-table gather, decode attention and
                   causal prefill-chunk attention (fp64)
                   (plus the same over an FP8 E4M3 cache)
  fp8              E4M3 codes: value table, round-to-nearest-even saturating encoding
  kv_memory        the KV-cache size formula and reservation-waste arithmetic

Every function is pinned by a test in tests/ against something other than
itself: closed forms, invariants stated by the pages (block placement does not
change the result, paged equals contiguous, shared prompt blocks equal private
copies, a copy-on-write step equals private sequences), a library attention
routine on special cases, a library FP8 conversion, or values the pages print.  Parity of the attention values is pinned only through those checks: the
pages print no attention outputs.
"""

from . import fp8, kv_memory, paged_attention  # noqa: F401
