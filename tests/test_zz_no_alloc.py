"""pa_decode_no_alloc, the decode entry point that allocates nothing (its scratch is the library's
fixed per-device array), against pa_decode, the entry point that takes a caller workspace.

Both run the same kernels, and with pa_decode's dynamic tail off they make the same static split,
so their outputs must be equal bit for bit; both must match the fp64 oracle within
|gpu - oracle| <= 1e-2 + 1e-2*|oracle|.  Two calls in a row share the one array: the second,
smaller batch must not see anything the first left there.
"""

import ctypes
import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_444_amd as pa
from helpers import (assert_close, cached_named_case, dev_i32, dev_u16, full_decode_oracle,
                     host_u16, upcast)
from oracle import paged_attention as oracle
from workloads import Spec, build_case

pytestmark = pytest.mark.gpu


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _args(case):
    d = case.decode
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    return (kc, vc, dev_u16(d.query), dev_i32(d.block_tables), dev_i32(d.seq_lens), d)


def _no_alloc_abi(case, kc, vc, q, bt, sl, d, out):
    """One pa_decode_no_alloc call through the C ABI (ctypes, raw device pointers)."""
    lib = pa.load_library()
    Hq, Hkv, D, bs = case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    st = lib.pa_decode_no_alloc(out.data_ptr(), q.data_ptr(), kc.data_ptr(), vc.data_ptr(),
                                case.num_blocks, bt.data_ptr(), sl.data_ptr(), d.num_seqs, Hq, Hkv,
                                D, bs, bt.shape[1], int(d.max_seq_len), ctypes.c_float(case.scale),
                                torch.cuda.current_stream().cuda_stream)
    assert st == 0, lib.pa_last_error()


def _workspace_decode(case, kc, vc, q, bt, sl, d):
    # pa_decode with the static split only (no dynamic tail), the split pa_decode_no_alloc makes
    with pa.tunables(PA_DECODE_TAIL_Q10=0):
        return pa.decode(q, kc, vc, bt, sl, num_kv_heads=case.num_kv_heads,
                         block_size=case.block_size, scale=float(case.scale),
                         max_seq_len=int(d.max_seq_len))


def test_no_alloc_equals_workspace_decode_on_two_calls():
    big = cached_named_case(2)  # 128 sequences, 64q/8kv, head_dim 128, lognormal lengths
    small = build_case(Spec(name="no_alloc_small", num_q_heads=16, num_kv_heads=2, head_dim=128,
                            block_size=32, seed=(444, 95),
                            decode_lens=[1, 40, 300, 17, 2049, 0, 129]))
    results = []
    for case in (big, small):
        say(f"no-alloc decode: {case.name}, B={case.decode.num_seqs}")
        kc, vc, q, bt, sl, d = _args(case)
        out = torch.full_like(q, 5.0)
        _no_alloc_abi(case, kc, vc, q, bt, sl, d, out)
        torch.cuda.synchronize()
        results.append((case, host_u16(out), host_u16(_workspace_decode(case, kc, vc, q, bt, sl, d))))
    (_, got_big, ref_big), (_, got_small, ref_small) = results
    assert np.array_equal(got_big, ref_big), "no-alloc decode differs from pa_decode (batch 128)"
    assert np.array_equal(got_small, ref_small), "no-alloc decode differs from pa_decode (small)"
    assert_close(upcast(got_big), full_decode_oracle(2), "no-alloc decode, 70B-shaped batch")
    d = small.decode
    ref = oracle.decode(d.query, small.key_cache, small.value_cache, d.block_tables, d.seq_lens,
                        small.num_kv_heads, small.head_dim, small.block_size, small.scale)
    assert_close(upcast(got_small), ref, "no-alloc decode, small batch after a large one")
    assert np.all(got_small[5] == 0)  # the zero-length sequence


def test_no_alloc_rejects_a_batch_larger_than_its_scratch():
    """4,096 sequences of the 70B shape need far more than the fixed scratch: the call returns
    PA_ERR_WORKSPACE on the host and launches nothing (the pointers are never dereferenced)."""
    lib = pa.load_library()
    out, q, kc, vc, bt, sl = ((k + 1) << 24 for k in range(6))  # distinct, aligned, never read
    st = lib.pa_decode_no_alloc(out, q, kc, vc, 100000, bt, sl, 4096, 64, 8, 128, 16, 512, 8192,
                                ctypes.c_float(0.088), None)
    assert st == 4
    assert b"pa_decode_no_alloc" in lib.pa_last_error()
