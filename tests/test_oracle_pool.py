"""The process-parallel oracle runner returns exactly what one direct oracle call returns."""

import numpy as np

from oracle import pool as oracle_pool
from oracle import fp8
from oracle import paged_attention as oracle
from workloads import Spec, build_case


def _case():
    return build_case(Spec(name="pool", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                           seed=(444, 90), decode_lens=[1, 40, 300, 17, 0, 129],
                           prefill=[(70, 33), (0, 20), (200, 5)]))


def test_parallel_prefill_rows_equal_one_call():
    c = _case()
    p = c.prefill
    rows = [0, 5, 32, 33, 40, 52, 57]
    direct = oracle.prefill_chunk(p.query, c.key_cache, c.value_cache, p.block_tables,
                                  p.query_start_loc, p.seq_lens, 2, 64, 16, c.scale, rows=rows)
    par = oracle_pool.prefill_rows("prefill_chunk", p.query, c.key_cache, c.value_cache,
                                   p.block_tables, p.query_start_loc, p.seq_lens, 2, 64, 16,
                                   c.scale, rows=rows)
    assert np.array_equal(par, direct)
    whole = oracle_pool.prefill_rows("prefill_chunk", p.query, c.key_cache, c.value_cache,
                                     p.block_tables, p.query_start_loc, p.seq_lens, 2, 64, 16,
                                     c.scale)
    assert np.array_equal(whole, oracle.prefill_chunk(p.query, c.key_cache, c.value_cache,
                                                      p.block_tables, p.query_start_loc,
                                                      p.seq_lens, 2, 64, 16, c.scale))


def test_parallel_decode_seqs_equal_one_call():
    c = _case()
    d = c.decode
    direct = oracle.decode(d.query, c.key_cache, c.value_cache, d.block_tables, d.seq_lens, 2, 64,
                           16, c.scale)
    par = oracle_pool.decode_seqs("decode", d.query, c.key_cache, c.value_cache, d.block_tables,
                                  d.seq_lens, 2, 64, 16, c.scale)
    assert np.array_equal(par, direct)
    kc8, vc8 = fp8.quantize(c.key_cache, 0.02), fp8.quantize(c.value_cache, 0.03)
    direct8 = oracle.decode_fp8(d.query, kc8, vc8, d.block_tables, d.seq_lens, 2, 64, 16, c.scale,
                                0.02, 0.03, seqs=[1, 3, 5])
    par8 = oracle_pool.decode_seqs("decode_fp8", d.query, kc8, vc8, d.block_tables, d.seq_lens, 2,
                                   64, 16, c.scale, seqs=[1, 3, 5], k_scale=0.02, v_scale=0.03)
    assert np.array_equal(par8, direct8[[1, 3, 5]])
