"""Pins for the fp64 CPU oracle (no GPU).

The oracle is checked against things other than itself: values the pages print,
closed forms of softmax attention, the invariants the pages state for paging
(physical placement is irrelevant, paged equals contiguous, shared prompt pages
equal private copies), a library attention routine on the same inputs, and
hand-computed offsets of the documented pool layout.  The last group plants
plausible mistakes in the oracle and checks that some pin catches each.
"""

import json
import math
import os

import numpy as np
import pytest
import torch

from oracle import kv_memory
from oracle import paged_attention as pa
from workloads import BlockAllocator, Spec, bf16_bits, build_case, build_cow_case, lognormal_lengths

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def small_case(seed=0, lens=(1, 7, 16, 17, 40, 95), Hq=8, Hkv=2, D=64, bs=16, **kw):
    return build_case(Spec(name="small", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                           block_size=bs, seed=(9, seed), decode_lens=list(lens), **kw))


def oracle_decode(case, **kw):
    d = case.decode
    return pa.decode(d.query, case.key_cache, case.value_cache, d.block_tables, d.seq_lens,
                     case.num_kv_heads, case.head_dim, case.block_size, case.scale, **kw)


# ---------------------------------------------------------------- printed values

def test_kv_memory_matches_printed_values():
    g = json.load(open(os.path.join(GOLDEN, "kv_memory.json")))
    e = g["llama3_70b_bytes_per_token"]
    assert kv_memory.kv_bytes_per_token(**e["args"]) == e["value"]
    e = g["llama3_70b_bytes_at_128k"]
    assert kv_memory.kv_bytes(**e["args"]) == e["value_gib"] * 2**30
    e = g["llama3_70b_bytes_at_4k"]
    assert kv_memory.kv_bytes(**e["args"]) == 1.25 * 2**30
    e = g["widehead_16x4x256_bytes_at_8192"]
    b = kv_memory.kv_bytes(**e["args"])
    assert b == 0.5 * 2**30 and round(b / 1e9, 2) == e["value_printed_gib"]
    e = g["reservation_waste_8192_at_1500"]
    assert round(100 * kv_memory.reservation_waste(**e["args"])) == e["value_printed_pct"]
    e = g["gqa_saving_64q_8kv"]
    full = kv_memory.kv_bytes_per_token(80, e["args"]["num_q_heads"], 128)
    gqa = kv_memory.kv_bytes_per_token(80, e["args"]["num_kv_heads"], 128)
    assert full // gqa == e["value"]


def test_paged_waste_below_printed_bound():
    # Exercise 4 of the serving lesson: 1,000 requests, mean 1,500, std 600, 16-token blocks.
    g = json.load(open(os.path.join(GOLDEN, "kv_memory.json")))
    lens = lognormal_lengths(np.random.default_rng(4), 1000)
    used = lens.sum()
    alloc = sum(-(-int(L) // 16) * 16 for L in lens)
    assert 100 * (1 - used / alloc) < g["paged_waste_below_pct"]["value"]
    reserved = 8192 * len(lens)
    assert 1 - used / reserved > 0.75  # the contiguous reservation wastes most of it
    assert kv_memory.paged_waste(17, 16) == pytest.approx(1 - 17 / 32)


# ---------------------------------------------------------------- inputs and bf16

def test_bf16_encoding_matches_torch():
    x = np.random.default_rng(1).standard_normal(100000, dtype=np.float32) * 10
    x[:4] = [0.0, -0.0, 1.0 + 2**-8, 1.0 + 3 * 2**-8]  # exact ties round to even
    ours = bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)
    back = pa.bf16_to_f64(ours)
    assert np.array_equal(back, torch.from_numpy(ref.view(np.int16)).view(torch.bfloat16).double().numpy())


def test_generator_is_deterministic():
    a, b = small_case(3), small_case(3)
    assert np.array_equal(a.key_cache, b.key_cache) and np.array_equal(a.decode.query, b.decode.query)
    assert np.array_equal(a.decode.block_tables, b.decode.block_tables)
    c = small_case(4)
    assert not np.array_equal(a.key_cache, c.key_cache)


def test_lognormal_moments():
    lens = lognormal_lengths(np.random.default_rng(0), 200000)
    assert abs(lens.mean() - 1500) < 10 and abs(lens.std() - 600) < 10
    assert lens.min() >= 16 and lens.max() <= 8192


def test_allocator_failure_modes():
    a = BlockAllocator(4, np.random.default_rng(0))
    ids = a.allocate(3)
    assert len(set(ids)) == 3 and a.num_free == 1
    with pytest.raises(MemoryError):
        a.allocate(2)
    a.share(ids[:1])
    a.release(ids[:1])
    assert a.refcount(ids[0]) == 1 and a.num_free == 1
    a.release(ids)
    assert a.num_free == 4
    with pytest.raises(ValueError):
        a.release(ids[:1])


# ---------------------------------------------------------------- layout and scatter

def test_pool_layout_hand_offsets():
    """The documented layout: K [blk][head][D/32 slice][16 tok][32], V [blk][head][D][16 tok],
    per 16-token sub-block.  Offsets below are worked out by hand for Hkv=2, D=64, bs=32."""
    Hkv, D, bs, N = 2, 64, 32, 3
    kc = np.zeros((N, Hkv * bs * D), np.uint16)
    vc = np.zeros_like(kc)
    key = np.zeros((1, Hkv, D), np.uint16)
    val = np.zeros_like(key)
    key[0, 1, 40] = 0x1234
    val[0, 1, 40] = 0x4321
    slot = np.array([1 * 32 + 17])  # block 1, offset 17: sub-block 1, token 1 of it
    kc2, vc2 = pa.reshape_and_cache(kc, vc, key, val, slot, Hkv, D, bs)
    # K: 4096 (block 1) + 2048 (head 1) + 1024 (sub-block 1) + 512 (slice 40//32=1) + 32 (token 1) + 8 (40%32)
    assert kc2.reshape(-1)[7720] == 0x1234 and np.count_nonzero(kc2) == 1
    # V: 4096 + 2048 + 1024 + 40*16 (dim 40) + 1 (token 1)
    assert vc2.reshape(-1)[7809] == 0x4321 and np.count_nonzero(vc2) == 1


def test_reshape_closed_form_and_round_trip():
    case = small_case(5, lens=(33, 64, 5), decode_new_token=True)
    r = case.reshape
    kc, vc = pa.reshape_and_cache(case.key_cache, case.value_cache, r.key, r.value, r.slot_mapping,
                                  case.num_kv_heads, case.head_dim, case.block_size)
    # Round trip: reading the written positions through the block tables returns the rows.
    d = case.decode
    for s, L in enumerate(d.seq_lens):
        k, v = pa.gather_kv(kc, vc, d.block_tables[s], int(L), case.num_kv_heads, case.head_dim,
                            case.block_size)
        assert np.array_equal(k[L - 1], pa.bf16_to_f64(r.key[s]))
        assert np.array_equal(v[L - 1], pa.bf16_to_f64(r.value[s]))
    # Closed form: exactly Hkv*D elements per written token changed in each pool (when the
    # new value differs from the old one), every other byte untouched.
    changed_k = np.count_nonzero(kc != case.key_cache)
    changed_v = np.count_nonzero(vc != case.value_cache)
    T = len(r.slot_mapping)
    assert changed_k <= T * case.num_kv_heads * case.head_dim
    assert changed_k > 0.9 * T * case.num_kv_heads * case.head_dim
    assert changed_v <= T * case.num_kv_heads * case.head_dim
    # Writing the old rows back restores the pool bit for bit.
    bs = case.block_size
    old_k = np.stack([pa.logical_blocks_k(case.key_cache, [s // bs], case.num_kv_heads,
                                          case.head_dim, bs)[0, :, s % bs] for s in r.slot_mapping])
    old_v = np.stack([pa.logical_blocks_v(case.value_cache, [s // bs], case.num_kv_heads,
                                          case.head_dim, bs)[0, :, s % bs] for s in r.slot_mapping])
    kc3, vc3 = pa.reshape_and_cache(kc, vc, old_k, old_v, r.slot_mapping, case.num_kv_heads,
                                    case.head_dim, bs)
    assert np.array_equal(kc3, case.key_cache) and np.array_equal(vc3, case.value_cache)


def test_reshape_skips_negative_and_rejects_bad_slots():
    case = small_case(6, lens=(20,), decode_new_token=True)
    r = case.reshape
    args = (case.num_kv_heads, case.head_dim, case.block_size)
    kc, vc = pa.reshape_and_cache(case.key_cache, case.value_cache, r.key, r.value,
                                  -np.ones_like(r.slot_mapping), *args)
    assert np.array_equal(kc, case.key_cache) and np.array_equal(vc, case.value_cache)
    with pytest.raises(ValueError):
        pa.reshape_and_cache(case.key_cache, case.value_cache, np.repeat(r.key, 2, 0),
                             np.repeat(r.value, 2, 0), np.repeat(r.slot_mapping, 2), *args)
    with pytest.raises(ValueError):
        pa.reshape_and_cache(case.key_cache, case.value_cache, r.key, r.value,
                             np.array([case.num_blocks * case.block_size]), *args)


# ---------------------------------------------------------------- attention closed forms

def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def test_single_key_returns_its_value():
    q, k, v = _rand((1, 4, 32), 0), _rand((1, 2, 32), 1), _rand((1, 2, 32), 2)
    out = pa.attention(q, k, v, 0.3)
    assert np.array_equal(out[0, :2], np.repeat(v[:, 0], 2, 0)) and np.array_equal(out[0, 2:], np.repeat(v[:, 1], 2, 0))


def test_zero_query_gives_mean_value():
    k, v = _rand((50, 2, 32), 1), _rand((50, 2, 32), 2)
    out = pa.attention(np.zeros((1, 4, 32)), k, v, 0.2)
    np.testing.assert_allclose(out[0, 1], v[:, 0].mean(0), rtol=1e-13, atol=1e-14)
    np.testing.assert_allclose(out[0, 3], v[:, 1].mean(0), rtol=1e-13, atol=1e-14)


def test_constant_values_and_equal_keys():
    q, k = _rand((3, 4, 16), 3), _rand((9, 1, 16), 4)
    v = np.broadcast_to(np.arange(16.0), (9, 1, 16)).copy()
    np.testing.assert_allclose(pa.attention(q, k, v, 0.5), np.broadcast_to(np.arange(16.0), (3, 4, 16)), rtol=1e-14)
    k_eq = np.broadcast_to(k[:1], k.shape).copy()
    v2 = _rand((9, 1, 16), 5)
    out = pa.attention(q[:1], k_eq, v2, 0.5)  # one row sees all 9 keys
    np.testing.assert_allclose(out[0, 0], v2[:, 0].mean(0), rtol=1e-13)


def test_sharp_query_selects_one_value():
    k = np.eye(8)[:, None, :]  # 8 orthonormal keys
    v = _rand((8, 1, 8), 6)
    q = 60.0 * k[5][None]       # aligned with key 5
    out = pa.attention(q, k, v, 1.0)
    np.testing.assert_allclose(out[0, 0], v[5, 0], atol=1e-20)


def test_output_is_convex_combination():
    q, k, v = _rand((5, 4, 16), 7), _rand((30, 2, 16), 8), _rand((30, 2, 16), 9)
    out = pa.attention(q, k, v, 0.25)
    for h in range(4):
        vv = v[:, h // 2]
        for i in range(5):
            vis = vv[:30 - 5 + i + 1]
            assert np.all(out[i, h] <= vis.max(0) + 1e-12) and np.all(out[i, h] >= vis.min(0) - 1e-12)


def _torch_reference(q, k, v, scale):
    """torch's scaled_dot_product_attention in float64 with an explicit bottom-right mask."""
    Tq, Hq, D = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    qt = torch.from_numpy(q).permute(1, 0, 2)
    kt = torch.from_numpy(k).permute(1, 0, 2).repeat_interleave(G, 0)
    vt = torch.from_numpy(v).permute(1, 0, 2).repeat_interleave(G, 0)
    mask = torch.arange(L)[None, :] <= (L - Tq + torch.arange(Tq))[:, None]
    o = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=mask, scale=float(scale))
    return o.permute(1, 0, 2).numpy()


@pytest.mark.parametrize("Tq,L,Hq,Hkv", [(1, 37, 8, 2), (5, 37, 8, 2), (16, 16, 4, 4), (7, 100, 6, 1)])
def test_matches_library_attention(Tq, L, Hq, Hkv):
    q, k, v = _rand((Tq, Hq, 32), 10), _rand((L, Hkv, 32), 11), _rand((L, Hkv, 32), 12)
    np.testing.assert_allclose(pa.attention(q, k, v, 0.17), _torch_reference(q, k, v, 0.17), rtol=1e-12, atol=1e-13)


def test_decode_matches_library_on_paged_case():
    case = small_case(7)
    out = oracle_decode(case)
    d = case.decode
    for s in range(d.num_seqs):
        k, v = pa.gather_kv(case.key_cache, case.value_cache, d.block_tables[s], int(d.seq_lens[s]),
                            case.num_kv_heads, case.head_dim, case.block_size)
        ref = _torch_reference(pa.bf16_to_f64(d.query[s])[None], k, v, case.scale)
        np.testing.assert_allclose(out[s], ref[0], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------- paging invariants

def _permute_blocks(case, seed):
    """Relabel physical blocks with a random permutation, moving contents and tables along."""
    N = case.num_blocks
    perm = np.random.default_rng(seed).permutation(N)  # old id -> new id
    kc = np.empty_like(case.key_cache)
    vc = np.empty_like(case.value_cache)
    kc[perm] = case.key_cache
    vc[perm] = case.value_cache
    return kc, vc, perm[case.decode.block_tables].astype(np.int32)


def test_block_permutation_changes_nothing():
    case = small_case(8)
    base = oracle_decode(case)
    kc, vc, bt = _permute_blocks(case, 1)
    d = case.decode
    out = pa.decode(d.query, kc, vc, bt, d.seq_lens, case.num_kv_heads, case.head_dim,
                    case.block_size, case.scale)
    assert np.array_equal(out, base)


def test_paged_equals_contiguous():
    """Fill an unpaged per-sequence cache by appending tokens in order (Step 1's KVCache),
    page the same tokens through reshape_and_cache, and compare."""
    rng = np.random.default_rng(13)
    Hq, Hkv, D, bs, L = 8, 2, 64, 16, 75
    k_tok = bf16_bits(rng.standard_normal((L, Hkv, D), dtype=np.float32))
    v_tok = bf16_bits(rng.standard_normal((L, Hkv, D), dtype=np.float32))
    q = bf16_bits(rng.standard_normal((1, Hq, D), dtype=np.float32))
    # contiguous cache: positions appended in order, read back [:end]
    k_contig = np.zeros((128, Hkv, D), np.uint16)
    v_contig = np.zeros_like(k_contig)
    k_contig[:L], v_contig[:L] = k_tok, v_tok
    ref = pa.contiguous_attention(pa.bf16_to_f64(q), pa.bf16_to_f64(k_contig[:L]),
                                  pa.bf16_to_f64(v_contig[:L]), 0.125)
    # paged: 5 blocks placed at scattered ids of a 40-block pool
    table = np.array([31, 2, 17, 8, 25], np.int32)
    slots = np.array([table[p // bs] * bs + p % bs for p in range(L)])
    kc = bf16_bits(rng.standard_normal((40, Hkv * bs * D), dtype=np.float32))
    vc = bf16_bits(rng.standard_normal((40, Hkv * bs * D), dtype=np.float32))
    kc, vc = pa.reshape_and_cache(kc, vc, k_tok, v_tok, slots, Hkv, D, bs)
    k, v = pa.gather_kv(kc, vc, table, L, Hkv, D, bs)
    assert np.array_equal(k, pa.bf16_to_f64(k_tok)) and np.array_equal(v, pa.bf16_to_f64(v_tok))
    out = pa.decode(q, kc, vc, table[None], np.array([L]), Hkv, D, bs, 0.125)
    assert np.array_equal(out[0], ref[0])


def test_prefix_sharing_equals_private_copies():
    groups = [([0, 1, 2], 32), ([3, 4], 48)]
    case = small_case(9, lens=(40, 33, 70, 60, 49), share_groups=groups)
    d = case.decode
    assert np.array_equal(d.block_tables[0, :2], d.block_tables[1, :2])
    base = oracle_decode(case)
    # give every sequence private copies of its shared blocks
    kc, vc = [case.key_cache], [case.value_cache]
    bt = d.block_tables.copy()
    nxt = case.num_blocks
    for members, shared in groups:
        for m in members:
            for j in range(shared // case.block_size):
                kc.append(case.key_cache[bt[m, j]][None])
                vc.append(case.value_cache[bt[m, j]][None])
                bt[m, j] = nxt
                nxt += 1
    kc, vc = np.concatenate(kc), np.concatenate(vc)
    out = pa.decode(d.query, kc, vc, bt, d.seq_lens, case.num_kv_heads, case.head_dim,
                    case.block_size, case.scale)
    assert np.array_equal(out, base)


def test_padding_and_unused_slots_never_read():
    case = small_case(10, lens=(5, 17, 33))
    base = oracle_decode(case)
    kc, vc = case.key_cache.copy(), case.value_cache.copy()
    used = set()
    d = case.decode
    for s, L in enumerate(d.seq_lens):
        used.update(d.block_tables[s, :-(-int(L) // case.block_size)].tolist())
    for b in range(case.num_blocks):
        if b not in used:
            kc[b] = 0x7FC0
            vc[b] = 0x7FC0
    # NaN into the unused tail slots of each sequence's last block
    bs = case.block_size
    for s, L in enumerate(d.seq_lens):
        L = int(L)
        tail = [d.block_tables[s, (L - 1) // bs] * bs + o for o in range(L % bs, bs)] if L % bs else []
        if tail:
            nan = np.full((len(tail), case.num_kv_heads, case.head_dim), 0x7FC0, np.uint16)
            kc, vc = pa.reshape_and_cache(kc, vc, nan, nan, np.array(tail), case.num_kv_heads,
                                          case.head_dim, bs)
    out = pa.decode(d.query, kc, vc, d.block_tables, d.seq_lens, case.num_kv_heads, case.head_dim,
                    bs, case.scale)
    assert np.array_equal(out, base)


# ---------------------------------------------------------------- chunking consistency

def _prefill_case(ctx, q_len, seed=11, **kw):
    return build_case(Spec(name="pf", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                           seed=(11, seed), prefill=[(ctx, q_len)], prefill_new_tokens=True, **kw))


def test_prefill_single_row_equals_decode_and_last_row():
    case = _prefill_case(45, 7)
    p = case.prefill
    args = (case.num_kv_heads, case.head_dim, case.block_size, case.scale)
    out = pa.prefill_chunk(p.query, case.key_cache, case.value_cache, p.block_tables,
                           p.query_start_loc, p.seq_lens, *args)
    # the last row of the chunk sees the whole context, like a decode at L = ctx + q_len
    dec = pa.decode(p.query[-1:], case.key_cache, case.value_cache, p.block_tables, p.seq_lens, *args)
    assert np.array_equal(out[-1], dec[0])
    # row i of the chunk equals a decode over the first ctx+i+1 keys
    dec3 = pa.decode(p.query[3:4], case.key_cache, case.value_cache, p.block_tables,
                     np.array([45 + 4]), *args)
    np.testing.assert_allclose(out[3], dec3[0], rtol=1e-13, atol=1e-15)


def test_consecutive_chunks_equal_one_causal_prefill():
    case = _prefill_case(0, 48, seed=12)
    p = case.prefill
    args = (case.num_kv_heads, case.head_dim, case.block_size, case.scale)
    whole = pa.prefill_chunk(p.query, case.key_cache, case.value_cache, p.block_tables,
                             p.query_start_loc, p.seq_lens, *args)
    parts = []
    for lo in range(0, 48, 16):  # three chunks of 16, each over everything before it
        parts.append(pa.prefill_chunk(p.query[lo:lo + 16], case.key_cache, case.value_cache,
                                      p.block_tables, np.array([0, 16]), np.array([lo + 16]), *args))
    np.testing.assert_allclose(np.concatenate(parts), whole, rtol=1e-13, atol=1e-15)
    # sampled rows equal the full computation
    rows = [0, 17, 47]
    np.testing.assert_allclose(pa.prefill_chunk(p.query, case.key_cache, case.value_cache,
                                                p.block_tables, p.query_start_loc, p.seq_lens,
                                                *args, rows=rows), whole[rows], rtol=0, atol=0)


def test_gqa_structure():
    q, k, v = _rand((1, 4, 16), 20), _rand((10, 2, 16), 21), _rand((10, 2, 16), 22)
    q[0, 1] = q[0, 0]
    out = pa.attention(q, k, v, 0.3)
    assert np.array_equal(out[0, 0], out[0, 1])  # same group, same query -> same output
    # G = 1 reduces to per-head attention
    q2 = _rand((1, 2, 16), 23)
    o2 = pa.attention(q2, k, v, 0.3)
    for h in range(2):
        np.testing.assert_allclose(o2[0, h], pa.attention(q2[:, h:h + 1], k[:, h:h + 1], v[:, h:h + 1], 0.3)[0, 0], rtol=1e-14)


def test_zero_length_sequence_gives_zeros():
    case = small_case(13, lens=(0, 5))
    out = oracle_decode(case)
    assert np.array_equal(out[0], np.zeros_like(out[0]))


# ---------------------------------------------------------------- copy-on-write

def test_copy_blocks_closed_form_and_rejections():
    rng = np.random.default_rng(21)
    kc = rng.integers(0, 1 << 16, size=(12, 2 * 16 * 64), dtype=np.uint16)
    vc = rng.integers(0, 1 << 16, size=(12, 2 * 16 * 64), dtype=np.uint16)
    m = np.array([[3, 7], [3, 9], [0, 11]])
    k2, v2 = pa.copy_blocks(kc, vc, m)
    for b in range(12):
        src = {7: 3, 9: 3, 11: 0}.get(b, b)
        assert np.array_equal(k2[b], kc[src]) and np.array_equal(v2[b], vc[src])
    # inputs are not modified; an empty mapping is the identity
    assert not np.array_equal(kc[7], kc[3])
    k3, v3 = pa.copy_blocks(kc, vc, np.zeros((0, 2), dtype=np.int64))
    assert np.array_equal(k3, kc) and np.array_equal(v3, vc)
    for bad in ([[1, 2], [3, 2]], [[1, 2], [2, 4]], [[1, 12]], [[-1, 2]]):
        with pytest.raises(ValueError):
            pa.copy_blocks(kc, vc, np.array(bad))


def test_cow_rule_keeps_refcounts():
    alloc = BlockAllocator(8)
    a = alloc.allocate(2)
    alloc.share(a)
    alloc.share(a)  # three holders
    t1, t2, t3 = list(a), list(a), list(a)
    p1 = alloc.prepare_write(t1, 20, 16)
    assert p1 == (a[1], t1[1]) and t1[0] == a[0] and alloc.refcount(a[1]) == 2
    assert alloc.refcount(t1[1]) == 1
    p2 = alloc.prepare_write(t2, 17, 16)
    assert p2 is not None and alloc.refcount(a[1]) == 1
    assert alloc.prepare_write(t3, 31, 16) is None and t3 == a  # last holder writes in place
    assert alloc.prepare_write(t1, 21, 16) is None  # already private
    assert alloc.num_free == 8 - 4


def _cow_expected(case):
    """Each candidate's decode output computed without any block copy: its K/V gathered from the
    pool as it was before the step through its table before the step, the new token appended."""
    d, r = case.decode, case.reshape
    Hkv, D, bs = case.num_kv_heads, case.head_dim, case.block_size
    out = np.zeros(d.query.shape)
    for b, table in enumerate(case.info["tables_before"]):
        L = int(d.seq_lens[b])
        k, v = pa.gather_kv(case.key_cache, case.value_cache, table, L - 1, Hkv, D, bs)
        k = np.concatenate([k, pa.bf16_to_f64(r.key[b])[None]])
        v = np.concatenate([v, pa.bf16_to_f64(r.value[b])[None]])
        out[b] = pa.attention(pa.bf16_to_f64(d.query[b])[None], k, v, case.scale)[0]
    return out


def _cow_step(case, copies):
    kc, vc = pa.copy_blocks(case.key_cache, case.value_cache, copies)
    r = case.reshape
    kc, vc = pa.reshape_and_cache(kc, vc, r.key, r.value, r.slot_mapping, case.num_kv_heads,
                                  case.head_dim, case.block_size)
    d = case.decode
    return pa.decode(d.query, kc, vc, d.block_tables, d.seq_lens, case.num_kv_heads,
                     case.head_dim, case.block_size, case.scale)


def test_cow_step_equals_private_sequences():
    # Two prompts of 37 tokens (the third 16-token block is partial) with four candidates each;
    # some candidates already diverged.  Copy-on-write must give every candidate exactly the
    # attention it would get with its own private cache.
    case, copies = build_cow_case("cow", 2, 4, 37, 8, 2, 64, 16, (444, 7),
                                  tails=[0, 0, 3, 11, 0, 5, 0, 20])
    assert len(copies) == 2
    assert np.array_equal(_cow_step(case, copies), _cow_expected(case))
    # Without the copies the candidates of a group would write the same slot.
    with pytest.raises(ValueError):
        _cow_step_without_copies(case)


def _cow_step_without_copies(case):
    d, r = case.decode, case.reshape
    bs = case.block_size
    slots = []
    for b, t in enumerate(case.info["tables_before"]):
        pos = int(d.seq_lens[b]) - 1
        blk = t[pos // bs] if pos // bs < len(t) else int(d.block_tables[b, pos // bs])
        slots.append(blk * bs + pos % bs)
    pa.reshape_and_cache(case.key_cache, case.value_cache, r.key, r.value, np.array(slots),
                         case.num_kv_heads, case.head_dim, case.block_size)


def test_cow_pin_catches_planted_copy_mistakes(monkeypatch):
    case, copies = build_cow_case("cow", 2, 4, 37, 8, 2, 64, 16, (444, 7),
                                  tails=[0, 0, 3, 11, 0, 5, 0, 20])
    want = _cow_expected(case)
    real = pa.copy_blocks

    def k_only(kc, vc, m):
        k2, _ = real(kc, vc, m)
        return k2, vc.copy()

    def reversed_pairs(kc, vc, m):
        return real(kc, vc, np.asarray(m)[:, ::-1])

    for fake in (k_only, reversed_pairs):
        with monkeypatch.context() as mp:
            mp.setattr(pa, "copy_blocks", fake)
            assert not np.array_equal(_cow_step(case, copies), want), fake.__name__


# ---------------------------------------------------------------- planted mistakes

def _pins_pass():
    """A compact run of the pins above; returns False if any fails."""
    try:
        test_matches_library_attention(5, 37, 8, 2)
        test_decode_matches_library_on_paged_case()
        test_pool_layout_hand_offsets()
        test_paged_equals_contiguous()
        test_prefill_single_row_equals_decode_and_last_row()
    except AssertionError:
        return False
    return True


def test_pins_pass_on_the_real_oracle():
    assert _pins_pass()


def test_pins_catch_planted_mistakes(monkeypatch):
    real_attention = pa.attention

    def no_scale(q, k, v, scale, rows=None):
        return real_attention(q, k, v, 1.0, rows)

    def wrong_group(q, k, v, scale, rows=None):
        Hq, Hkv = q.shape[1], k.shape[1]
        perm = [(h % Hkv) * (Hq // Hkv) + h // Hkv for h in range(Hq)]  # h % Hkv mapping
        return real_attention(q[:, np.argsort(perm)], k, v, scale, rows)[:, perm]

    def causal_off_by_one(q, k, v, scale, rows=None):
        if q.shape[0] == 1:
            return real_attention(q, k, v, scale, rows)
        return real_attention(q, k[:-1], v[:-1], scale, rows)

    def plain_k_layout(pool, ids, Hkv, D, bs):  # token-major K inside a block
        return pool.reshape(-1, Hkv, bs, D)[np.asarray(ids)]

    for name, fake in [("attention", no_scale), ("attention", wrong_group),
                       ("attention", causal_off_by_one), ("logical_blocks_k", plain_k_layout)]:
        with monkeypatch.context() as m:
            m.setattr(pa, name, fake)
            assert not _pins_pass(), f"planted mistake {fake.__name__} went unnoticed"


# ---------------------------------------------------------------- scalar brute force

def _bf16_scalar(bits):
    import struct
    return struct.unpack("<f", struct.pack("<I", int(bits) << 16))[0]


def _scalar_kv(pool, b, h, o, d, Hkv, D, bs, kind):
    """One cached element, read through the documented block layout (not the oracle's views)."""
    tile = (b * Hkv + h) * bs * D
    if kind == "k":
        off = (o // 16) * 16 * D + (d // 32) * 512 + (o % 16) * 32 + d % 32
    else:
        off = (o // 16) * 16 * D + d * 16 + o % 16
    return _bf16_scalar(pool.reshape(-1)[tile + off])


def _scalar_attention(q_row, table, L, last_key, kc, vc, kvh, Hkv, D, bs, scale):
    """softmax(scale * q.k) . v over keys 0..last_key, with plain loops and math.exp."""
    scores = []
    for p in range(last_key + 1):
        b, o = int(table[p // bs]), p % bs
        scores.append(scale * sum(q_row[d] * _scalar_kv(kc, b, kvh, o, d, Hkv, D, bs, "k")
                                  for d in range(D)))
    m = max(scores)
    w = [math.exp(s - m) for s in scores]
    tot = sum(w)
    out = []
    for d in range(D):
        acc = 0.0
        for p in range(last_key + 1):
            b, o = int(table[p // bs]), p % bs
            acc += w[p] * _scalar_kv(vc, b, kvh, o, d, Hkv, D, bs, "v")
        out.append(acc / tot)
    return out


def test_oracle_matches_scalar_loops_on_tiny_cases():
    # decode: four sequences over two blocks sizes' worth of positions, GQA 2
    case = small_case(31, lens=(1, 7, 17, 40), Hq=4, Hkv=2, D=64, bs=16)
    d = case.decode
    ref = oracle_decode(case)
    scale = float(case.scale)
    for s in range(4):
        L = int(d.seq_lens[s])
        for h in range(4):
            q_row = [_bf16_scalar(x) for x in d.query[s, h]]
            got = _scalar_attention(q_row, d.block_tables[s], L, L - 1, case.key_cache,
                                    case.value_cache, h // 2, 2, 64, 16, scale)
            assert np.allclose(got, ref[s, h], rtol=1e-12, atol=1e-12)
    # prefill chunk: 5 rows after 20 cached tokens, 32-token blocks, causal by loop bounds
    case = build_case(Spec(name="p", num_q_heads=2, num_kv_heads=1, head_dim=32, block_size=32,
                           seed=(32,), prefill=[(20, 5)]))
    p = case.prefill
    ref = pa.prefill_chunk(p.query, case.key_cache, case.value_cache, p.block_tables,
                           p.query_start_loc, p.seq_lens, 1, 32, 32, case.scale)
    for t in range(5):
        for h in range(2):
            q_row = [_bf16_scalar(x) for x in p.query[t, h]]
            got = _scalar_attention(q_row, p.block_tables[0], 25, 20 + t, case.key_cache,
                                    case.value_cache, 0, 1, 32, 32, float(case.scale))
            assert np.allclose(got, ref[t, h], rtol=1e-12, atol=1e-12)
