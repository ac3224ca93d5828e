"""Seeded synthetic inputs for paged KV-cache attention (test and benchmark harness).

This package is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It draws random numbers, encodes them as bf16, samples sequence
lengths and hands out physical blocks; it holds none of the attention
arithmetic and knows nothing about how a block is laid out inside: pools are
produced as flat arrays of bf16 bit patterns, one row per physical block.
"""

from .inputs import (  # noqa: F401
    BlockAllocator,
    Case,
    DecodeBatch,
    PrefillBatch,
    ReshapeBatch,
    Spec,
    bf16_bits,
    build_case,
    build_cow_case,
    lognormal_lengths,
    named_case,
    NAMED_CASES,
    tp_share_case,
)
