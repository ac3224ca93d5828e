"""GPU parity of pa_prefill_chunk (chunked-prefill attention on matrix cores) against the fp64
CPU oracle.

Every output element must satisfy |gpu - oracle| <= 1e-2 + 1e-2*|oracle|, on every row of every
shape, the 32k-context workload included (its oracle rows are computed on several host
processes).  GPU-side invariants (block relabelling, NaN in
never-read memory, repeated runs) must hold bitwise.
"""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_444_amd as pa
from helpers import (assert_close, cached_named_case, dev_i32, dev_i64, dev_u16,
                     full_prefill_oracle, host_u16, oracle_pools_after_reshape, upcast)
from oracle import paged_attention as oracle
from workloads import Spec, build_case

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_reshape(case, kc, vc):
    r = case.reshape
    pa.reshape_and_cache(dev_u16(r.key), dev_u16(r.value), kc, vc, dev_i64(r.slot_mapping),
                         num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                         block_size=case.block_size)


def gpu_prefill(case, kc, vc, block_tables=None, query=None):
    p = case.prefill
    bt = p.block_tables if block_tables is None else block_tables
    q = p.query if query is None else query
    out = pa.prefill_chunk(dev_u16(q), kc, vc, dev_i32(bt), dev_i32(p.query_start_loc),
                           dev_i32(p.seq_lens), num_kv_heads=case.num_kv_heads,
                           block_size=case.block_size, max_q_len=p.max_q_len,
                           max_seq_len=p.max_seq_len, scale=float(case.scale))
    torch.cuda.synchronize()
    return host_u16(out)


def oracle_prefill(case, kc, vc, rows=None):
    p = case.prefill
    return oracle.prefill_chunk(p.query, kc, vc, p.block_tables, p.query_start_loc, p.seq_lens,
                                case.num_kv_heads, case.head_dim, case.block_size, case.scale,
                                rows=rows)


def small_case(chunks, Hq=8, Hkv=2, D=64, bs=16, seed=40):
    """chunks: list of (prior context, chunk length); the chunk's K/V is written by reshape."""
    return build_case(Spec(name="prefill", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                           block_size=bs, seed=(seed, Hq, Hkv, D, bs), prefill=chunks,
                           prefill_new_tokens=True))


# ------------------------------------------------------------------------- 32k-context chunk

def test_prefill_parity_long_context_chunk():
    """512-token chunk over 31,744 cached tokens (64q/8kv, D 128, 16-token blocks): the chunked
    prefill part of the mixed workload, with the chunk's own K/V written by reshape first."""
    case = cached_named_case(4)
    p = case.prefill
    say(f"prefill cfg4: {case.name}, q_len={p.max_q_len}, L={p.max_seq_len}")
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    gpu_reshape(case, kc, vc)
    got = upcast(gpu_prefill(case, kc, vc))
    ref = full_prefill_oracle(4)
    assert ref.shape == got.shape
    # every row: all 32 query tiles of the chunk, both context splits, all 64 heads
    assert_close(got, ref, "prefill 512-token chunk over 31,744 cached tokens")


# ------------------------------------------------------------------------- shapes and edges

SHAPES = [
    # (Hq, Hkv, D, bs)
    (8, 2, 64, 16),
    (16, 1, 64, 32),
    (4, 4, 128, 16),
    (64, 8, 128, 16),
    (16, 2, 128, 32),
    (16, 4, 256, 32),
    (2, 2, 256, 16),
]
CHUNKS = [(0, 1), (0, 37), (70, 33), (5, 16), (511, 2), (1000, 129), (3, 300), (40, 512)]


@pytest.mark.parametrize("Hq,Hkv,D,bs", SHAPES)
def test_prefill_shapes_and_ragged_chunks(Hq, Hkv, D, bs):
    say(f"prefill shape Hq={Hq} Hkv={Hkv} D={D} bs={bs}")
    case = small_case(CHUNKS, Hq, Hkv, D, bs)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    gpu_reshape(case, kc, vc)
    got = upcast(gpu_prefill(case, kc, vc))
    okc, ovc = oracle_pools_after_reshape(case)
    assert_close(got, oracle_prefill(case, okc, ovc), "prefill ragged chunks")


@pytest.mark.parametrize("splits", ["1", "3", "7"])
def test_prefill_context_splits(splits):
    """The context split changes only how key ranges are spread over workgroups."""
    case = small_case([(4000, 200), (2500, 64), (0, 300)], Hq=16, Hkv=2, D=128, bs=16, seed=42)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    gpu_reshape(case, kc, vc)
    with pa.tunables(PA_PREFILL_SPLITS=int(splits)):
        a = gpu_prefill(case, kc, vc)
        b = gpu_prefill(case, kc, vc)
    assert np.array_equal(a, b)
    okc, ovc = oracle_pools_after_reshape(case)
    assert_close(upcast(a), oracle_prefill(case, okc, ovc), f"prefill with {splits} splits")


def test_prefill_single_row_matches_decode():
    """A one-token chunk is a decode step: both kernels must match the oracle on the same input."""
    case = small_case([(700, 1), (33, 1), (0, 1)], Hq=64, Hkv=8, D=128, bs=16, seed=43)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    gpu_reshape(case, kc, vc)
    got_p = upcast(gpu_prefill(case, kc, vc))
    p = case.prefill
    got_d = upcast(host_u16(pa.decode(dev_u16(p.query), kc, vc, dev_i32(p.block_tables),
                                      dev_i32(p.seq_lens), num_kv_heads=8, block_size=16,
                                      scale=float(case.scale), max_seq_len=p.max_seq_len)))
    okc, ovc = oracle_pools_after_reshape(case)
    ref = oracle_prefill(case, okc, ovc)
    assert_close(got_p, ref, "prefill q_len=1")
    assert_close(got_d, ref, "decode of the same rows")


def test_prefill_empty_and_zero_length_chunks():
    case = small_case([(50, 20), (10, 0), (0, 5)], seed=44)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    gpu_reshape(case, kc, vc)
    got = upcast(gpu_prefill(case, kc, vc))
    okc, ovc = oracle_pools_after_reshape(case)
    assert_close(got, oracle_prefill(case, okc, ovc), "prefill with an empty chunk")
    q = torch.empty((0, 8, 64), dtype=torch.bfloat16, device="cuda")
    out = pa.prefill_chunk(q, kc, vc, torch.zeros((0, 1), dtype=torch.int32, device="cuda"),
                           torch.zeros(1, dtype=torch.int32, device="cuda"),
                           torch.zeros(0, dtype=torch.int32, device="cuda"), num_kv_heads=2,
                           block_size=16, max_q_len=0, max_seq_len=0)
    assert out.shape == (0, 8, 64)


# ------------------------------------------------------------------------- invariants on the GPU

def test_prefill_block_permutation_and_nan_never_read():
    case = small_case([(300, 70), (1029, 100)], Hq=16, Hkv=2, D=128, bs=16, seed=45)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    gpu_reshape(case, kc, vc)
    base = gpu_prefill(case, kc, vc)
    assert np.array_equal(base, gpu_prefill(case, kc, vc))
    okc, ovc = oracle_pools_after_reshape(case)
    # relabel every physical block
    perm = np.random.default_rng(6).permutation(case.num_blocks)
    pk, pv = np.empty_like(okc), np.empty_like(ovc)
    pk[perm], pv[perm] = okc, ovc
    got = gpu_prefill(case, dev_u16(pk), dev_u16(pv), block_tables=perm[case.prefill.block_tables])
    assert np.array_equal(got, base)
    # NaN in every unused block and in the slots past each sequence's end
    p = case.prefill
    bs = case.block_size
    used = set()
    for s, L in enumerate(p.seq_lens):
        used.update(p.block_tables[s, :-(-int(L) // bs)].tolist())
    nk, nv = okc.copy(), ovc.copy()
    unused = [b for b in range(case.num_blocks) if b not in used]
    nk[unused] = 0x7FC0
    nv[unused] = 0x7FC0
    kc2, vc2 = dev_u16(nk), dev_u16(nv)
    tail = []
    for s, L in enumerate(p.seq_lens):
        L = int(L)
        if L % bs:
            tail += [int(p.block_tables[s, (L - 1) // bs]) * bs + o for o in range(L % bs, bs)]
    nan = np.full((len(tail), case.num_kv_heads, case.head_dim), 0x7FC0, np.uint16)
    pa.reshape_and_cache(dev_u16(nan), dev_u16(nan), kc2, vc2, dev_i64(np.array(tail)),
                         num_kv_heads=case.num_kv_heads, head_dim=case.head_dim, block_size=bs)
    assert np.array_equal(gpu_prefill(case, kc2, vc2), base)


def test_prefill_abi_rejects_bad_arguments():
    case = small_case([(30, 10)], seed=46)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    p = case.prefill
    q = dev_u16(p.query)
    bt, qsl, sl = dev_i32(p.block_tables), dev_i32(p.query_start_loc), dev_i32(p.seq_lens)
    out = torch.full_like(q, 3.0)
    before = out.clone()
    with pytest.raises(pa.PagedAttentionError) as e:  # Hq % Hkv
        pa.prefill_chunk(q, kc, vc, bt, qsl, sl, num_kv_heads=3, block_size=16, max_q_len=10,
                         max_seq_len=40, out=out)
    assert e.value.status == 2
    with pytest.raises(pa.PagedAttentionError) as e:  # max_q_len > max_seq_len
        pa.prefill_chunk(q, kc, vc, bt, qsl, sl, num_kv_heads=2, block_size=16, max_q_len=50,
                         max_seq_len=40, out=out)
    assert e.value.status == 2
    with pytest.raises(pa.PagedAttentionError) as e:  # unsupported block size
        pa.prefill_chunk(q, kc, vc, bt, qsl, sl, num_kv_heads=2, block_size=8, max_q_len=10,
                         max_seq_len=40, out=out)
    assert e.value.status == 3
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), before.view(torch.int16))
