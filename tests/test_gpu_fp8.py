"""GPU parity of the FP8 (E4M3) KV cache: pa_reshape_and_cache_fp8 and pa_decode_fp8 against the
fp64 CPU oracle.

Reshape must reproduce the oracle's byte pools bit for bit (the codes are integers decided in fp32
on both sides).  Decode over FP8 pools quantised by the oracle must satisfy
|gpu - oracle| <= 1e-2 + 1e-2*|oracle| element by element, the oracle attending over the
dequantised cache.  Widening every finite code to bf16 must be exact.
"""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_444_amd as pa
from helpers import (FP8_K_SCALE, FP8_V_SCALE, assert_close, cached_fp8_pools, cached_named_case,
                     dev_i32, dev_i64, dev_u16, dev_u8, full_decode_oracle, full_prefill_oracle,
                     host_u16, host_u8, oracle_quantize_pool, upcast)
from oracle import fp8
from oracle import paged_attention as oracle
from workloads import Spec, build_case

pytestmark = pytest.mark.gpu

# Per-tensor scales for N(0,1) caches: the largest of ~10^8 normal draws (about 6) maps near 448.
K_SCALE = FP8_K_SCALE
V_SCALE = FP8_V_SCALE


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _gpu_reshape_fp8(case, kc8, vc8, k_scale, v_scale):
    r = case.reshape
    pa.reshape_and_cache_fp8(dev_u16(r.key), dev_u16(r.value), kc8, vc8, dev_i64(r.slot_mapping),
                             num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                             block_size=case.block_size, k_scale=k_scale, v_scale=v_scale)
    torch.cuda.synchronize()


@pytest.mark.parametrize("cfg,k_scale,v_scale", [
    (1, K_SCALE, V_SCALE),
    (1, 1e-3, 100.0),   # K saturates at 448, V lands in the subnormal range
    (4, K_SCALE, V_SCALE),
    (5, 0.25, 3.0),
])
def test_reshape_fp8_bit_exact(cfg, k_scale, v_scale):
    case = cached_named_case(cfg)
    say(f"reshape fp8 cfg{cfg}: T={len(case.reshape.slot_mapping)} scales {k_scale}, {v_scale}")
    rng = np.random.default_rng((444, 70, cfg))
    kc8 = rng.integers(0, 256, size=case.key_cache.shape, dtype=np.uint8)
    vc8 = rng.integers(0, 256, size=case.value_cache.shape, dtype=np.uint8)
    gk, gv = dev_u8(kc8), dev_u8(vc8)
    _gpu_reshape_fp8(case, gk, gv, k_scale, v_scale)
    r = case.reshape
    ok, ov = oracle.reshape_and_cache_fp8(kc8, vc8, r.key, r.value, r.slot_mapping,
                                          case.num_kv_heads, case.head_dim, case.block_size,
                                          k_scale, v_scale)
    assert np.array_equal(host_u8(gk), ok) and np.array_equal(host_u8(gv), ov)


def test_every_finite_code_widens_exactly():
    # One-token sequences: the output of each is v_scale * V[0] rounded to bf16, which is exact
    # for v_scale = 1 since every E4M3 value is a bf16 value.  Four sequences cover the 254
    # finite codes (and two repeats) over 64 head dimensions.
    Hkv, D, bs = 1, 64, 16
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)] + [0x00, 0x80],
                     dtype=np.uint8).reshape(4, 64)
    kc8 = np.zeros((4, Hkv * bs * D), dtype=np.uint8)
    vc8 = np.zeros((4, Hkv * bs * D), dtype=np.uint8)
    for b in range(4):
        vc8[b].reshape(bs // 16, D, 16)[0, :, 0] = codes[b]  # token 0 of block b, V layout [D][16]
    q = np.zeros((4, 1, D), dtype=np.uint16)
    out = pa.decode_fp8(dev_u16(q), dev_u8(kc8), dev_u8(vc8), dev_i32(np.arange(4)[:, None]),
                        dev_i32(np.ones(4)), num_kv_heads=1, block_size=bs, k_scale=1.0,
                        v_scale=1.0, max_seq_len=1)
    torch.cuda.synchronize()
    got = upcast(host_u16(out)).reshape(4, 64)
    want = fp8.decode(codes)
    assert np.array_equal(got, want)
    # and through the oracle's own FP8 path
    ref = oracle.decode_fp8(q, kc8, vc8, np.arange(4)[:, None], np.ones(4, dtype=np.int32), 1, D,
                            bs, 0.125, 1.0, 1.0)
    assert np.array_equal(ref[:, 0], want)


def _fp8_case_pools(cfg):
    """A named workload with its pools after the step's reshape (bf16, by the oracle), quantised
    whole by the oracle's quantiser."""
    kc8, vc8 = cached_fp8_pools(cfg)
    return cached_named_case(cfg), kc8, vc8


@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_decode_fp8_parity_named(cfg):
    case, kc8, vc8 = _fp8_case_pools(cfg)
    d = case.decode
    say(f"decode fp8 cfg{cfg}: {case.name}, B={d.num_seqs}, max L={d.max_seq_len}")
    gk, gv = dev_u8(kc8), dev_u8(vc8)
    kw = dict(num_kv_heads=case.num_kv_heads, block_size=case.block_size, k_scale=K_SCALE,
              v_scale=V_SCALE, scale=float(case.scale), max_seq_len=d.max_seq_len)
    out = pa.decode_fp8(dev_u16(d.query), gk, gv, dev_i32(d.block_tables), dev_i32(d.seq_lens), **kw)
    out2 = pa.decode_fp8(dev_u16(d.query), gk, gv, dev_i32(d.block_tables), dev_i32(d.seq_lens), **kw)
    torch.cuda.synchronize()
    got = host_u16(out)
    assert np.array_equal(got, host_u16(out2)), "FP8 decode is not reproducible"
    # every sequence of the batch
    assert_close(upcast(got), full_decode_oracle(cfg, fp8=True), f"FP8 decode cfg{cfg}")


@pytest.mark.parametrize("Hq,Hkv,D,bs", [(8, 2, 64, 16), (16, 1, 64, 32), (4, 4, 128, 16),
                                         (16, 2, 128, 32), (8, 2, 256, 16)])
def test_decode_fp8_shapes_and_ragged_lengths(Hq, Hkv, D, bs):
    lens = [1, 15, 16, 17, 33, 100, 257, 1000, 0, 2049]
    case = build_case(Spec(name="fp8", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                           seed=(444, 72, Hq, Hkv, D, bs), decode_lens=lens))
    kc8 = oracle_quantize_pool(case.key_cache, 0.02)
    vc8 = oracle_quantize_pool(case.value_cache, 0.03)
    d = case.decode
    out = pa.decode_fp8(dev_u16(d.query), dev_u8(kc8), dev_u8(vc8), dev_i32(d.block_tables),
                        dev_i32(d.seq_lens), num_kv_heads=Hkv, block_size=bs, k_scale=0.02,
                        v_scale=0.03, scale=float(case.scale), max_seq_len=d.max_seq_len)
    torch.cuda.synchronize()
    ref = oracle.decode_fp8(d.query, kc8, vc8, d.block_tables, d.seq_lens, Hkv, D, bs, case.scale,
                            0.02, 0.03)
    assert_close(upcast(host_u16(out)), ref, f"FP8 decode {Hq}/{Hkv}/{D}/{bs}")


def _gpu_prefill_fp8(case, kc8, vc8, k_scale, v_scale):
    p = case.prefill
    out = pa.prefill_chunk_fp8(dev_u16(p.query), dev_u8(kc8), dev_u8(vc8), dev_i32(p.block_tables),
                               dev_i32(p.query_start_loc), dev_i32(p.seq_lens),
                               num_kv_heads=case.num_kv_heads, block_size=case.block_size,
                               max_q_len=p.max_q_len, max_seq_len=p.max_seq_len, k_scale=k_scale,
                               v_scale=v_scale, scale=float(case.scale))
    torch.cuda.synchronize()
    return host_u16(out)


def test_prefill_fp8_parity_long_context_chunk():
    """The mixed workload's 512-token chunk over 31,744 cached tokens, over an FP8 cache."""
    case, kc8, vc8 = _fp8_case_pools(4)
    p = case.prefill
    say(f"prefill fp8 cfg4: q_len={p.max_q_len}, L={p.max_seq_len}")
    got = upcast(_gpu_prefill_fp8(case, kc8, vc8, K_SCALE, V_SCALE))
    # every row: all 32 query tiles, both context splits, all 64 heads
    assert_close(got, full_prefill_oracle(4, fp8=True),
                 "FP8 prefill 512-token chunk over 31,744 cached tokens")


@pytest.mark.parametrize("Hq,Hkv,D,bs", [(8, 2, 64, 16), (16, 1, 64, 32), (64, 8, 128, 16),
                                         (16, 2, 128, 32), (16, 4, 256, 32), (2, 2, 256, 16)])
def test_prefill_fp8_shapes_and_ragged_chunks(Hq, Hkv, D, bs):
    chunks = [(0, 1), (0, 37), (70, 33), (5, 16), (1000, 129), (40, 512)]
    case = build_case(Spec(name="fp8p", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                           seed=(444, 75, Hq, Hkv, D, bs), prefill=chunks))
    kc8 = oracle_quantize_pool(case.key_cache, 0.02)
    vc8 = oracle_quantize_pool(case.value_cache, 0.03)
    got = upcast(_gpu_prefill_fp8(case, kc8, vc8, 0.02, 0.03))
    p = case.prefill
    ref = oracle.prefill_chunk_fp8(p.query, kc8, vc8, p.block_tables, p.query_start_loc,
                                   p.seq_lens, Hkv, D, bs, case.scale, 0.02, 0.03)
    assert_close(got, ref, f"FP8 prefill {Hq}/{Hkv}/{D}/{bs}")


def test_fp8_nan_in_unused_slots_never_read():
    """NaN codes (0x7F) in every slot past each sequence's length, in its last block and in all
    unreferenced blocks, must not change decode or prefill outputs (bitwise)."""
    Hkv, D, bs = 2, 64, 16
    case = build_case(Spec(name="fp8nan", num_q_heads=8, num_kv_heads=Hkv, head_dim=D,
                           block_size=bs, seed=(444, 76), decode_lens=[1, 15, 17, 40, 95],
                           prefill=[(30, 7), (0, 20)]))
    kc8 = oracle_quantize_pool(case.key_cache, 0.02)
    vc8 = oracle_quantize_pool(case.value_cache, 0.03)
    used = {}
    d, p = case.decode, case.prefill
    for tables, lens in ((d.block_tables, d.seq_lens), (p.block_tables, p.seq_lens)):
        for row, L in zip(tables, lens):
            for pos in range(int(L)):
                used.setdefault(int(row[pos // bs]), set()).add(pos % bs)
    kn, vn = kc8.copy(), vc8.copy()
    for b in range(kc8.shape[0]):
        for o in range(bs):
            if o in used.get(b, ()):
                continue
            for h in range(Hkv):
                kv = kn[b].reshape(Hkv, bs // 16, D // 32, 16, 32)
                vv = vn[b].reshape(Hkv, bs // 16, D, 16)
                kv[h, o // 16, :, o % 16, :] = 0x7F
                vv[h, o // 16, :, o % 16] = 0x7F

    def run(k, v):
        dec = pa.decode_fp8(dev_u16(d.query), dev_u8(k), dev_u8(v), dev_i32(d.block_tables),
                            dev_i32(d.seq_lens), num_kv_heads=Hkv, block_size=bs, k_scale=0.02,
                            v_scale=0.03, scale=float(case.scale), max_seq_len=d.max_seq_len)
        pre = pa.prefill_chunk_fp8(dev_u16(p.query), dev_u8(k), dev_u8(v), dev_i32(p.block_tables),
                                   dev_i32(p.query_start_loc), dev_i32(p.seq_lens),
                                   num_kv_heads=Hkv, block_size=bs, max_q_len=p.max_q_len,
                                   max_seq_len=p.max_seq_len, k_scale=0.02, v_scale=0.03,
                                   scale=float(case.scale))
        torch.cuda.synchronize()
        return host_u16(dec), host_u16(pre)

    a_dec, a_pre = run(kc8, vc8)
    b_dec, b_pre = run(kn, vn)
    assert np.array_equal(a_dec, b_dec) and np.array_equal(a_pre, b_pre)
    assert not np.isnan(upcast(b_dec)).any() and not np.isnan(upcast(b_pre)).any()
