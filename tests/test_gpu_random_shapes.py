"""Seeded random sweep: decode and chunked prefill, bf16 and FP8 caches, against the oracle.

Each case draws a supported shape (head_dim 64/128/256, a power-of-two group with
group * head_dim <= 1024, 1-8 KV heads, 16- or 32-token blocks) and a length mix:
- decode lengths of 1, block_size - 1, block_size and block_size + 1, plus lognormal lengths;
- one to three prefill chunks (prior context 0-1,500 tokens, chunk 1-200 tokens).
Each decode sequence's new token and each chunk's own K/V are written by reshape first. Outputs
must satisfy |gpu - oracle| <= 1e-2 + 1e-2*|oracle| element by element; reshape must match bit for bit.
"""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_444_amd as pa
from helpers import (assert_close, dev_i32, dev_i64, dev_u16, dev_u8, host_u16,
                     oracle_pools_after_reshape, oracle_quantize_pool, upcast)
from oracle import paged_attention as oracle
from workloads import Spec, build_case

pytestmark = pytest.mark.gpu

K_SCALE, V_SCALE = 6.0 / 448, 5.5 / 448


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def draw_case(seed):
    rng = np.random.default_rng((444, 90, seed))
    D = int(rng.choice([64, 128, 256]))
    G = int(rng.choice([g for g in (1, 2, 4, 8, 16) if g * D <= 1024]))
    Hkv = int(rng.choice([1, 2, 4, 8] if G <= 4 else [1, 2, 4]))
    bs = int(rng.choice([16, 32]))
    n_dec = int(rng.integers(1, 9))
    edges = [1, bs - 1, bs, bs + 1]
    lens = [int(rng.choice(edges)) if rng.random() < 0.4 else
            int(np.clip(np.rint(rng.lognormal(6.5, 0.8)), 1, 3000)) for _ in range(n_dec)]
    chunks = [(int(rng.integers(0, 1501)), int(rng.integers(1, 201)))
              for _ in range(int(rng.integers(1, 4)))]
    spec = Spec(name=f"random{seed}", num_q_heads=G * Hkv, num_kv_heads=Hkv, head_dim=D,
                block_size=bs, seed=(444, 91, seed), decode_lens=lens, decode_new_token=True,
                prefill=chunks, prefill_new_tokens=True)
    return build_case(spec)


@pytest.mark.parametrize("seed", range(12))
def test_random_shapes_and_lengths(seed):
    case = draw_case(seed)
    Hkv, D, bs = case.num_kv_heads, case.head_dim, case.block_size
    d, p, r = case.decode, case.prefill, case.reshape
    say(f"random case {seed}: Hq={case.num_q_heads} Hkv={Hkv} D={D} bs={bs} "
        f"decode L={d.seq_lens.tolist()} chunks q={np.diff(p.query_start_loc).tolist()} "
        f"L={p.seq_lens.tolist()}")
    kw = dict(num_kv_heads=Hkv, block_size=bs)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    pa.reshape_and_cache(dev_u16(r.key), dev_u16(r.value), kc, vc, dev_i64(r.slot_mapping),
                         head_dim=D, **kw)
    okc, ovc = oracle_pools_after_reshape(case)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(kc).reshape(okc.shape), okc), "reshape (K)"
    assert np.array_equal(host_u16(vc).reshape(ovc.shape), ovc), "reshape (V)"

    out = pa.decode(dev_u16(d.query), kc, vc, dev_i32(d.block_tables), dev_i32(d.seq_lens),
                    scale=float(case.scale), max_seq_len=d.max_seq_len, **kw)
    ref = oracle.decode(d.query, okc, ovc, d.block_tables, d.seq_lens, Hkv, D, bs, case.scale)
    assert_close(upcast(host_u16(out)), ref, f"decode, random case {seed}")

    outp = pa.prefill_chunk(dev_u16(p.query), kc, vc, dev_i32(p.block_tables),
                            dev_i32(p.query_start_loc), dev_i32(p.seq_lens), max_q_len=p.max_q_len,
                            max_seq_len=p.max_seq_len, scale=float(case.scale), **kw)
    refp = oracle.prefill_chunk(p.query, okc, ovc, p.block_tables, p.query_start_loc, p.seq_lens,
                                Hkv, D, bs, case.scale)
    assert_close(upcast(host_u16(outp)), refp, f"prefill, random case {seed}")

    k8, v8 = oracle_quantize_pool(okc, K_SCALE), oracle_quantize_pool(ovc, V_SCALE)
    g8k, g8v = dev_u8(k8), dev_u8(v8)
    kw8 = dict(kw, k_scale=K_SCALE, v_scale=V_SCALE)
    out8 = pa.decode_fp8(dev_u16(d.query), g8k, g8v, dev_i32(d.block_tables), dev_i32(d.seq_lens),
                         scale=float(case.scale), max_seq_len=d.max_seq_len, **kw8)
    ref8 = oracle.decode_fp8(d.query, k8, v8, d.block_tables, d.seq_lens, Hkv, D, bs, case.scale,
                             K_SCALE, V_SCALE)
    assert_close(upcast(host_u16(out8)), ref8, f"FP8 decode, random case {seed}")

    outp8 = pa.prefill_chunk_fp8(dev_u16(p.query), g8k, g8v, dev_i32(p.block_tables),
                                 dev_i32(p.query_start_loc), dev_i32(p.seq_lens),
                                 max_q_len=p.max_q_len, max_seq_len=p.max_seq_len,
                                 scale=float(case.scale), **kw8)
    refp8 = oracle.prefill_chunk_fp8(p.query, k8, v8, p.block_tables, p.query_start_loc,
                                     p.seq_lens, Hkv, D, bs, case.scale, K_SCALE, V_SCALE)
    assert_close(upcast(host_u16(outp8)), refp8, f"FP8 prefill, random case {seed}")
