"""GPU parity of pa_copy_blocks and of a whole copy-on-write step against the fp64 CPU oracle.

Copies must reproduce the oracle's pool images bit for bit.  In the copy-on-write step (copy the
shared partial prompt block for each diverging candidate, write the new tokens, decode), the pools
must match bit for bit and the decode outputs must satisfy |gpu - oracle| <= 1e-2 + 1e-2*|oracle|.
"""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_444_amd as pa
from helpers import assert_close, dev_i32, dev_i64, dev_u16, host_u16, upcast
from oracle import paged_attention as oracle
from workloads import build_cow_case

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _random_pools(n_blocks, elems, seed):
    rng = np.random.default_rng(seed)
    kc = rng.integers(0, 1 << 16, size=(n_blocks, elems), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(n_blocks, elems), dtype=np.uint16)
    return kc, vc


@pytest.mark.parametrize("Hkv,D,bs,n_blocks,n_pairs", [
    (2, 64, 16, 64, 1),
    (8, 128, 16, 512, 200),
    (4, 256, 32, 96, 33),
    (1, 64, 16, 80001, 40000),  # more work items than the grid: the grid-stride loop
])
def test_copy_blocks_bit_exact(Hkv, D, bs, n_blocks, n_pairs):
    say(f"copy_blocks Hkv={Hkv} D={D} bs={bs} blocks={n_blocks} pairs={n_pairs}")
    kc, vc = _random_pools(n_blocks, Hkv * bs * D, (444, 60, n_pairs))
    rng = np.random.default_rng((444, 61, n_pairs))
    ids = rng.permutation(n_blocks)
    m = np.stack([ids[:n_pairs], ids[n_pairs:2 * n_pairs]], axis=1).astype(np.int64)
    okc, ovc = oracle.copy_blocks(kc, vc, m)
    gk, gv = dev_u16(kc), dev_u16(vc)
    pa.copy_blocks(gk, gv, dev_i64(m), num_kv_heads=Hkv, head_dim=D, block_size=bs)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(gk), okc) and np.array_equal(host_u16(gv), ovc)


def test_copy_blocks_skips_pairs_outside_the_pool_and_empty_calls():
    Hkv, D, bs, n = 2, 128, 16, 40
    kc, vc = _random_pools(n, Hkv * bs * D, (444, 62))
    m = np.array([[3, 7], [-1, 9], [5, 40], [41, 11], [0, 12]], dtype=np.int64)
    okc, ovc = oracle.copy_blocks(kc, vc, m[[0, 4]])
    gk, gv = dev_u16(kc), dev_u16(vc)
    pa.copy_blocks(gk, gv, dev_i64(m), num_kv_heads=Hkv, head_dim=D, block_size=bs)
    pa.copy_blocks(gk, gv, dev_i64(np.zeros((0, 2))), num_kv_heads=Hkv, head_dim=D, block_size=bs)
    torch.cuda.synchronize()
    assert np.array_equal(host_u16(gk), okc) and np.array_equal(host_u16(gv), ovc)


def _gpu_cow_step(case, copies):
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    kw = dict(num_kv_heads=case.num_kv_heads, head_dim=case.head_dim, block_size=case.block_size)
    pa.copy_blocks(kc, vc, dev_i64(copies), **kw)
    r = case.reshape
    pa.reshape_and_cache(dev_u16(r.key), dev_u16(r.value), kc, vc, dev_i64(r.slot_mapping), **kw)
    d = case.decode
    out = pa.decode(dev_u16(d.query), kc, vc, dev_i32(d.block_tables), dev_i32(d.seq_lens),
                    num_kv_heads=case.num_kv_heads, block_size=case.block_size,
                    scale=float(case.scale), max_seq_len=d.max_seq_len)
    torch.cuda.synchronize()
    return host_u16(kc), host_u16(vc), host_u16(out)


@pytest.mark.parametrize("prompts,cands,prompt_len,Hq,Hkv,D,bs,tails", [
    (2, 4, 37, 8, 2, 64, 16, [0, 0, 3, 11, 0, 5, 0, 20]),
    (3, 5, 70, 16, 4, 256, 32, None),
    # Rollouts of 8 prompts x 16 candidates at the Llama-3.3-70B shape; the 4,100-token prompt
    # ends 4 tokens into its 257th block, which every candidate writing at 4,100 must copy.
    (8, 16, 4100, 64, 8, 128, 16, None),
    (8, 16, 4100, 64, 8, 128, 16, "random"),
])
def test_cow_step_parity(prompts, cands, prompt_len, Hq, Hkv, D, bs, tails):
    if tails == "random":
        tails = np.random.default_rng((444, 63)).integers(0, 1025, size=prompts * cands).tolist()
    case, copies = build_cow_case("cow", prompts, cands, prompt_len, Hq, Hkv, D, bs, (444, 64),
                                  tails=tails)
    say(f"cow step {prompts}x{cands} prompt {prompt_len} D={D}: {len(copies)} copies")
    gk, gv, out = _gpu_cow_step(case, copies)
    okc, ovc = oracle.copy_blocks(case.key_cache, case.value_cache, copies)
    r = case.reshape
    okc, ovc = oracle.reshape_and_cache(okc, ovc, r.key, r.value, r.slot_mapping, Hkv, D, bs)
    assert np.array_equal(gk, okc) and np.array_equal(gv, ovc)
    d = case.decode
    ref = oracle.decode(d.query, okc, ovc, d.block_tables, d.seq_lens, Hkv, D, bs, case.scale)
    assert_close(upcast(out), ref, "decode after the copy-on-write step")
