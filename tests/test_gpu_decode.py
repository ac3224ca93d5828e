"""GPU parity of pa_reshape_and_cache and pa_decode against the fp64 CPU oracle.

reshape_and_cache must reproduce the oracle's pool images bit for bit; decode outputs must satisfy
|gpu - oracle| <= 1e-2 + 1e-2*|oracle| element by element.  GPU-side invariants (block relabelling,
shared prompt blocks vs private copies, repeated runs, NaN in never-read memory) must hold bitwise.
"""

import sys

import numpy as np
import pytest
import torch

import paged_kv_cache_444_amd as pa
from helpers import (assert_close, cached_named_case, cached_oracle_pools, cached_tp_share_case,
                     dev_i32, dev_i64, dev_u16, full_decode_oracle, full_tp_share_oracle, host_u16,
                     oracle_pools_after_reshape, upcast)
from oracle import paged_attention as oracle
from workloads import Spec, build_case

pytestmark = pytest.mark.gpu


@pytest.fixture
def tune():
    """Set library tunables for one test; the previous values come back afterwards."""
    saved = {}

    def set_(name, value):
        saved.setdefault(name, pa.get_tunable(name))
        pa.set_tunable(name, int(value))

    yield set_
    for k, v in saved.items():
        pa.set_tunable(k, v)

# bf16 decode steps: "0" the vector step, "1" the matrix-core step (the default).
STEPS = ["0", "1"]


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def gpu_reshape(case, kc, vc):
    r = case.reshape
    pa.reshape_and_cache(dev_u16(r.key), dev_u16(r.value), kc, vc, dev_i64(r.slot_mapping),
                         num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                         block_size=case.block_size)


def gpu_decode(case, kc, vc, block_tables=None, seq_lens=None, query=None):
    d = case.decode
    bt = d.block_tables if block_tables is None else block_tables
    sl = d.seq_lens if seq_lens is None else seq_lens
    q = d.query if query is None else query
    out = pa.decode(dev_u16(q), kc, vc, dev_i32(bt), dev_i32(sl), num_kv_heads=case.num_kv_heads,
                    block_size=case.block_size, scale=float(case.scale),
                    max_seq_len=int(np.max(sl)) if len(sl) else 0)
    torch.cuda.synchronize()
    return host_u16(out)


def oracle_decode(case, kc, vc, seqs=None):
    d = case.decode
    return oracle.decode(d.query, kc, vc, d.block_tables, d.seq_lens, case.num_kv_heads,
                         case.head_dim, case.block_size, case.scale, seqs=seqs)


# ------------------------------------------------------------------------- named workloads

@pytest.mark.parametrize("cfg", [1, 4, 5])
def test_reshape_bit_exact_named(cfg):
    case = cached_named_case(cfg)
    say(f"reshape cfg{cfg}: {case.name}, T={len(case.reshape.slot_mapping)}")
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    gpu_reshape(case, kc, vc)
    torch.cuda.synchronize()
    ok_k, ok_v = cached_oracle_pools(cfg)
    assert np.array_equal(host_u16(kc).reshape(ok_k.shape), ok_k)
    assert np.array_equal(host_u16(vc).reshape(ok_v.shape), ok_v)


@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_decode_parity_named(cfg):
    case = cached_named_case(cfg)
    d = case.decode
    say(f"decode cfg{cfg}: {case.name}, B={d.num_seqs}, max L={d.max_seq_len}")
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    if case.reshape is not None:
        gpu_reshape(case, kc, vc)
    got = upcast(gpu_decode(case, kc, vc))
    # every sequence of the batch (the oracle runs on several host processes)
    assert_close(got, full_decode_oracle(cfg), f"decode cfg{cfg}")


@pytest.mark.parametrize("step", STEPS)
def test_decode_parity_tp8_share(step, tune):
    """One GPU's share of the 70B-shaped batch-128 decode at tensor parallelism 8 over KV heads:
    8 query heads on 1 KV head, the same 128 lognormal lengths.  With one KV head the workgroup
    head-quad split is off and every sequence is spread over several waves, so this runs the
    per-wave split and the merge of many pieces per sequence."""
    case = cached_tp_share_case(8)
    d = case.decode
    say(f"decode TP=8 share: {case.name}, Hq={case.num_q_heads}, Hkv={case.num_kv_heads}")
    tune("PA_DECODE_MFMA", step)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    a = gpu_decode(case, kc, vc)
    assert np.array_equal(a, gpu_decode(case, kc, vc)), "not reproducible"
    assert_close(upcast(a), full_tp_share_oracle(8), f"decode, TP=8 share ({step})")


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
EDGE_LENS = [1, 2, 15, 16, 17, 31, 33, 255, 511, 512, 513, 1023, 1024, 1025, 1537, 3000]


@pytest.mark.parametrize("Hq,Hkv,D,bs", SHAPES)
def test_decode_shapes_and_ragged_lengths(Hq, Hkv, D, bs):
    say(f"decode shape Hq={Hq} Hkv={Hkv} D={D} bs={bs}")
    case = build_case(Spec(name="edge", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                           seed=(21, Hq, Hkv, D, bs), decode_lens=EDGE_LENS, decode_new_token=True))
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    gpu_reshape(case, kc, vc)
    got = upcast(gpu_decode(case, kc, vc))
    okc, ovc = oracle_pools_after_reshape(case)
    assert_close(got, oracle_decode(case, okc, ovc), "decode edge lengths")


def test_decode_zero_length_and_empty_batch():
    case = build_case(Spec(name="zero", num_q_heads=8, num_kv_heads=2, head_dim=128, block_size=16,
                           seed=(22,), decode_lens=[0, 5, 0, 700]))
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    got = gpu_decode(case, kc, vc)
    assert np.all(got[0] == 0) and np.all(got[2] == 0)
    assert_close(upcast(got), oracle_decode(case, case.key_cache, case.value_cache), "zero-length rows")
    # empty batch is a no-op
    q = torch.empty((0, 8, 128), dtype=torch.bfloat16, device="cuda")
    out = pa.decode(q, kc, vc, torch.zeros((0, 1), dtype=torch.int32, device="cuda"),
                    torch.zeros(0, dtype=torch.int32, device="cuda"), num_kv_heads=2, block_size=16,
                    max_seq_len=0)
    assert out.shape == (0, 8, 128)


def test_decode_max_length_and_scale():
    """Longest context the workloads produce (8,192) plus a non-default scale."""
    case = build_case(Spec(name="long", num_q_heads=64, num_kv_heads=8, head_dim=128, block_size=16,
                           seed=(23,), decode_lens=[8192, 8191, 4097]))
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    d = case.decode
    out = pa.decode(dev_u16(d.query), kc, vc, dev_i32(d.block_tables), dev_i32(d.seq_lens),
                    num_kv_heads=8, block_size=16, scale=0.3, max_seq_len=8192)
    ref = oracle.decode(d.query, case.key_cache, case.value_cache, d.block_tables, d.seq_lens, 8, 128,
                        16, np.float32(0.3))
    assert_close(upcast(host_u16(out)), ref, "decode at 8192 tokens, scale 0.3")


def test_decode_many_short_sequences_and_wide_batch():
    """Several hundred sequences (more than one 256-wide scan chunk), lengths 0..70, so that one
    wave's range crosses many units and most units sit inside a single wave."""
    lens = np.random.default_rng(24).integers(0, 71, size=700).tolist()
    case = build_case(Spec(name="short", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                           seed=(24,), decode_lens=lens))
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    got = upcast(gpu_decode(case, kc, vc))
    assert_close(got, oracle_decode(case, case.key_cache, case.value_cache), "700 short sequences")


@pytest.mark.parametrize("max_len", [16, 64])
def test_decode_one_unit_per_worker(max_len):
    """A batch of 128 sequences of one to four steps at the 70B head shape: the plan gives every
    unit its own workgroup (no partial slots, no merge work) and must still match the oracle."""
    lens = np.random.default_rng((24, max_len)).integers(1, max_len + 1, size=128).tolist()
    case = build_case(Spec(name="oneunit", num_q_heads=64, num_kv_heads=8, head_dim=128,
                           block_size=16, seed=(25, max_len), decode_lens=lens))
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    got = upcast(gpu_decode(case, kc, vc))
    assert_close(got, oracle_decode(case, case.key_cache, case.value_cache),
                 f"128 sequences of at most {max_len} tokens")


@pytest.mark.parametrize("step", STEPS)
@pytest.mark.parametrize("workers", [4, 12, 64])
def test_decode_few_workers_long_ranges(workers, step, tune):
    """Few worker waves: each wave streams hundreds of steps, crossing the 64-block id window and
    several unit boundaries; results must not depend on the worker count beyond rounding."""
    case = build_case(Spec(name="few", num_q_heads=16, num_kv_heads=4, head_dim=128, block_size=16,
                           seed=(25,), decode_lens=[3000, 1, 2049, 4100, 17, 1500]))
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    tune("PA_DECODE_WORKERS", str(workers))
    tune("PA_DECODE_MFMA", step)
    got = upcast(gpu_decode(case, kc, vc))
    assert_close(got, oracle_decode(case, case.key_cache, case.value_cache), f"{workers} workers")


@pytest.mark.parametrize("step", STEPS)
@pytest.mark.parametrize("static_q10,chunk", [(1024, 4), (768, 4), (512, 1), (640, 16)])
def test_decode_static_and_dynamic_splits(static_q10, chunk, step, tune):
    """The share of statically split steps and the dynamic chunk size change only how work is
    handed out: every split must match the oracle, and one workspace is reused across calls."""
    case = cached_named_case(2)
    tune("PA_DECODE_STATIC_Q10", str(static_q10))
    tune("PA_DECODE_CHUNK", str(chunk))
    tune("PA_DECODE_MFMA", step)
    d = case.decode
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    q, bt, sl = dev_u16(d.query), dev_i32(d.block_tables), dev_i32(d.seq_lens)
    ws = torch.zeros(pa.decode_workspace_bytes(d.num_seqs, case.num_q_heads, case.num_kv_heads,
                                               case.head_dim, d.max_seq_len),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        out = pa.decode(q, kc, vc, bt, sl, num_kv_heads=case.num_kv_heads, block_size=16,
                        scale=float(case.scale), max_seq_len=d.max_seq_len, workspace=ws)
        outs.append(host_u16(out))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0])  # deterministic whatever wave takes which chunk
    assert_close(upcast(outs[0]), full_decode_oracle(2),
                 f"decode static {static_q10}/1024, chunk {chunk}")


@pytest.mark.parametrize("Hq,Hkv,D,bs", [(16, 1, 64, 16), (8, 2, 128, 32), (8, 2, 256, 16),
                                          (4, 4, 128, 16)])
@pytest.mark.parametrize("chunk", [1, 3, 16])
@pytest.mark.parametrize("step", STEPS)
def test_decode_shared_chunks_shapes(Hq, Hkv, D, bs, chunk, step, tune):
    """Dynamic chunks are shared by a workgroup's waves (some idle when a piece has fewer steps
    than waves) and combined in LDS: every head shape must match the oracle, deterministically."""
    case = build_case(Spec(name="shared", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                           block_size=bs, seed=(26, Hq, D, bs),
                           decode_lens=[1, 17, 300, 1000, 2049, 5, 640]))
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    tune("PA_DECODE_WORKERS", "8")
    tune("PA_DECODE_STATIC_Q10", "600")
    tune("PA_DECODE_CHUNK", str(chunk))
    tune("PA_DECODE_MFMA", step)
    a = gpu_decode(case, kc, vc)
    assert np.array_equal(a, gpu_decode(case, kc, vc))
    assert_close(upcast(a), oracle_decode(case, case.key_cache, case.value_cache),
                 f"shared chunks of {chunk} steps")


@pytest.mark.parametrize("Hq,Hkv,D,bs,workers", [(32, 8, 128, 16, None), (16, 4, 256, 32, "8"),
                                                 (32, 8, 64, 16, "12"), (8, 2, 128, 16, None),
                                                 (16, 4, 128, 32, "4")])
@pytest.mark.parametrize("step", STEPS)
def test_decode_head_quads(Hq, Hkv, D, bs, workers, step, tune):
    """Workgroup workers over units of four KV heads (a wave per head, the four reading the same
    block together) change only how steps are handed out: every shape must match the oracle,
    deterministically, with the merge kernel combining units split between workgroups."""
    case = build_case(Spec(name="quads", num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                           block_size=bs, seed=(28, Hq, D, bs),
                           decode_lens=[1, 17, 300, 1000, 2049, 5, 640, 0, 3000]))
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    tune("PA_DECODE_QUAD", "1")
    tune("PA_DECODE_MFMA", step)
    if workers:
        tune("PA_DECODE_WORKERS", workers)
    a = gpu_decode(case, kc, vc)
    assert np.array_equal(a, gpu_decode(case, kc, vc))
    assert_close(upcast(a), oracle_decode(case, case.key_cache, case.value_cache),
                 "decode over head quads")


@pytest.mark.parametrize("cfg", [2, 5])
def test_decode_head_quads_named(cfg, tune):
    case = cached_named_case(cfg)
    d = case.decode
    tune("PA_DECODE_QUAD", "1")
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    if case.reshape is not None:
        gpu_reshape(case, kc, vc)
    got = upcast(gpu_decode(case, kc, vc))
    assert_close(got, full_decode_oracle(cfg), f"decode over head quads, workload {cfg}")


@pytest.mark.parametrize("quad", ["0", "1"])
@pytest.mark.parametrize("piece_cost,workers", [("0", None), ("1", "8"), ("6", None), ("64", "12"),
                                                ("64", None)])
def test_decode_piece_cost_split(quad, piece_cost, workers, tune):
    """The static split weighs every unit a worker starts as extra steps.  Any weight (clamped to
    half a worker's share of steps) must still give each worker a non-empty range, owners that the
    merge agrees with, and the oracle's result, with many short and empty sequences between long
    ones."""
    case = build_case(Spec(name="piece_cost", num_q_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=16, seed=(29, int(piece_cost)),
                           decode_lens=[1, 0, 17, 2000, 3, 16, 0, 33, 700, 1, 1, 4100, 250, 0, 9]))
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    tune("PA_DECODE_QUAD", quad)
    tune("PA_DECODE_PIECE_COST", piece_cost)
    if workers:
        tune("PA_DECODE_WORKERS", workers)
    say(f"decode piece cost {piece_cost}, quad {quad}, workers {workers}")
    a = gpu_decode(case, kc, vc)
    assert np.array_equal(a, gpu_decode(case, kc, vc))
    assert_close(upcast(a), oracle_decode(case, case.key_cache, case.value_cache),
                 f"decode with piece cost {piece_cost}")


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("tail_q10,chunk", [(0, 12), (160, 12), (512, 1), (300, 64), (160, 3),
                                            (512, 256)])
def test_decode_dynamic_tail(tail_q10, chunk, fp8, tune):
    """The head-quad split with its last steps handed out as claimed chunks: whichever
    workgroup takes a chunk, the result must be the same bit for bit on every call (fixed partial
    slots, merged in chunk order) and match the oracle; many short, empty and long sequences."""
    lens = np.random.default_rng((444, 91)).integers(0, 3000, size=40).tolist()
    lens[3] = lens[17] = 0
    lens[5] = 1
    case = build_case(Spec(name="tail", num_q_heads=32, num_kv_heads=8, head_dim=128,
                           block_size=16, seed=(444, 92, tail_q10, chunk), decode_lens=lens))
    d = case.decode
    tune("PA_DECODE_TAIL_Q10_FP8" if fp8 else "PA_DECODE_TAIL_Q10", tail_q10)
    tune("PA_DECODE_TAIL_CHUNK", chunk)
    say(f"decode dynamic tail {tail_q10}/1024, chunk {chunk}, fp8 {fp8}")
    if fp8:
        from helpers import dev_u8, oracle_quantize_pool

        kc8 = oracle_quantize_pool(case.key_cache, 0.02)
        vc8 = oracle_quantize_pool(case.value_cache, 0.03)
        gk, gv = dev_u8(kc8), dev_u8(vc8)

        def run():
            out = pa.decode_fp8(dev_u16(d.query), gk, gv, dev_i32(d.block_tables),
                                dev_i32(d.seq_lens), num_kv_heads=8, block_size=16, k_scale=0.02,
                                v_scale=0.03, scale=float(case.scale), max_seq_len=d.max_seq_len)
            torch.cuda.synchronize()
            return host_u16(out)

        ref = oracle.decode_fp8(d.query, kc8, vc8, d.block_tables, d.seq_lens, 8, 128, 16,
                                case.scale, 0.02, 0.03)
    else:
        kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)

        def run():
            return gpu_decode(case, kc, vc)

        ref = oracle_decode(case, case.key_cache, case.value_cache)
    a = run()
    for _ in range(3):
        assert np.array_equal(a, run()), "the dynamic tail changed the result between calls"
    assert_close(upcast(a), ref, f"decode with a dynamic tail of {tail_q10}/1024")


@pytest.mark.parametrize("tail_q10,chunk", [(64, 8), (160, 4)])
def test_decode_dynamic_tail_named(tail_q10, chunk, tune):
    """The dynamic tail at the 70B batch-128 shape (every CU's workgroup claims chunks near the end
    of its static range): the same bits on every call and every sequence matching the oracle."""
    case = cached_named_case(2)
    tune("PA_DECODE_TAIL_Q10", tail_q10)
    tune("PA_DECODE_TAIL_CHUNK", chunk)
    say(f"decode dynamic tail {tail_q10}/1024, chunk {chunk}, 70B batch 128")
    d = case.decode
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    q, bt, sl = dev_u16(d.query), dev_i32(d.block_tables), dev_i32(d.seq_lens)
    ws = torch.zeros(pa.decode_workspace_bytes(d.num_seqs, case.num_q_heads, case.num_kv_heads,
                                               case.head_dim, d.max_seq_len),
                     dtype=torch.uint8, device="cuda")
    outs = []
    for _ in range(3):
        out = pa.decode(q, kc, vc, bt, sl, num_kv_heads=case.num_kv_heads, block_size=16,
                        scale=float(case.scale), max_seq_len=d.max_seq_len, workspace=ws)
        outs.append(host_u16(out))
    for o in outs[1:]:
        assert np.array_equal(o, outs[0]), "the dynamic tail changed the result between calls"
    assert_close(upcast(outs[0]), full_decode_oracle(2),
                 f"decode with a dynamic tail of {tail_q10}/1024 at the 70B shape")


def test_decode_workspace_sizes_on_device():
    n = pa.decode_workspace_bytes(128, 64, 8, 128, 8192)
    assert n >= 128 * 8 * 8 * (128 + 2) * 4  # at least one partial slot per unit
    assert pa.decode_workspace_bytes(128, 64, 8, 128, 16) == n  # independent of lengths
    assert pa.decode_workspace_bytes(256, 64, 8, 128, 8192) > n


# ------------------------------------------------------------------------- invariants on the GPU

def _small(seed=30, **kw):
    args = dict(name="inv", num_q_heads=16, num_kv_heads=2, head_dim=128, block_size=16,
                seed=(seed,), decode_lens=[3, 100, 513, 1200, 47])
    args.update(kw)
    return build_case(Spec(**args))


def test_decode_block_permutation_bitwise():
    case = _small()
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    base = gpu_decode(case, kc, vc)
    perm = np.random.default_rng(5).permutation(case.num_blocks)
    pk = np.empty_like(case.key_cache)
    pv = np.empty_like(case.value_cache)
    pk[perm], pv[perm] = case.key_cache, case.value_cache
    got = gpu_decode(case, dev_u16(pk), dev_u16(pv), block_tables=perm[case.decode.block_tables])
    assert np.array_equal(got, base)


def test_decode_prefix_sharing_bitwise():
    # The shared tables make the kernel use ordinary loads and the private copies streaming
    # (non-temporal) loads, so this also checks that the load kind never changes the result.
    groups = [([0, 1, 2], 512), ([3, 4], 256)]
    case = _small(31, decode_lens=[600, 513, 1100, 300, 257], share_groups=groups)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    base = gpu_decode(case, kc, vc)
    bt = case.decode.block_tables.copy()
    extra_k, extra_v = [case.key_cache], [case.value_cache]
    nxt = case.num_blocks
    for members, shared in groups:
        for m in members:
            for j in range(shared // case.block_size):
                extra_k.append(case.key_cache[bt[m, j]][None])
                extra_v.append(case.value_cache[bt[m, j]][None])
                bt[m, j] = nxt
                nxt += 1
    got = gpu_decode(case, dev_u16(np.concatenate(extra_k)), dev_u16(np.concatenate(extra_v)),
                     block_tables=bt)
    assert np.array_equal(got, base)


def test_decode_deterministic_and_nan_never_read():
    case = _small(32)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    a = gpu_decode(case, kc, vc)
    b = gpu_decode(case, kc, vc)
    assert np.array_equal(a, b)
    # NaN into every unused block and into the tail slots past each sequence's end
    d = case.decode
    bs = case.block_size
    used = set()
    for s, L in enumerate(d.seq_lens):
        used.update(d.block_tables[s, :-(-int(L) // bs)].tolist())
    pk, pv = case.key_cache.copy(), case.value_cache.copy()
    unused = [b for b in range(case.num_blocks) if b not in used]
    pk[unused] = 0x7FC0
    pv[unused] = 0x7FC0
    kc2, vc2 = dev_u16(pk), dev_u16(pv)
    tail = []
    for s, L in enumerate(d.seq_lens):
        L = int(L)
        if L % bs:
            tail += [int(d.block_tables[s, (L - 1) // bs]) * bs + o for o in range(L % bs, bs)]
    nan = np.full((len(tail), case.num_kv_heads, case.head_dim), 0x7FC0, np.uint16)
    pa.reshape_and_cache(dev_u16(nan), dev_u16(nan), kc2, vc2, dev_i64(np.array(tail)),
                         num_kv_heads=case.num_kv_heads, head_dim=case.head_dim, block_size=bs)
    c = gpu_decode(case, kc2, vc2)
    assert np.array_equal(c, a)


# ------------------------------------------------------------------------- ABI error paths

def test_abi_rejects_bad_arguments_without_touching_buffers():
    case = _small(33)
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    d = case.decode
    q = dev_u16(d.query)
    bt, sl = dev_i32(d.block_tables), dev_i32(d.seq_lens)
    out = torch.full_like(q, 7.0)
    before = out.clone()
    with pytest.raises(pa.PagedAttentionError) as e:  # Hq % Hkv != 0
        pa.decode(q, kc, vc, bt, sl, num_kv_heads=3, block_size=16, max_seq_len=2000, out=out)
    assert e.value.status == 2
    with pytest.raises(pa.PagedAttentionError) as e:  # unsupported block size
        pa.decode(q, kc, vc, bt, sl, num_kv_heads=2, block_size=8, max_seq_len=1200, out=out)
    assert e.value.status == 3
    with pytest.raises(pa.PagedAttentionError) as e:  # max_seq_len beyond the table width
        pa.decode(q, kc, vc, bt, sl, num_kv_heads=2, block_size=16,
                  max_seq_len=bt.shape[1] * 16 + 1, out=out)
    assert e.value.status == 2
    with pytest.raises(pa.PagedAttentionError) as e:  # workspace too small
        pa.decode(q, kc, vc, bt, sl, num_kv_heads=2, block_size=16, max_seq_len=1200, out=out,
                  workspace=torch.empty(16, dtype=torch.uint8, device="cuda"))
    assert e.value.status == 4
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), before.view(torch.int16))
    lib = pa.load_library()
    assert lib.pa_decode(0, 0, 0, 0, 1000, 0, 0, 1, 8, 2, 128, 16, 4, 64, 0.1, 0, 0, 0) == 1


# ------------------------------------------------------------------------- matrix-core step

@pytest.mark.parametrize("step", ["0", "1"])
@pytest.mark.parametrize("cfg", [1, 2, 3, 5])
def test_decode_vector_and_matrix_core_steps_named(cfg, step, tune):
    """The bf16 decode on each step against the oracle: the vector step (PA_DECODE_MFMA=0) and the
    matrix-core step (the default, and the one FP8 pools always use)."""
    tune("PA_DECODE_MFMA", step)
    case = cached_named_case(cfg)
    d = case.decode
    say(f"decode (step {step}) cfg{cfg}: {case.name}, B={d.num_seqs}, max L={d.max_seq_len}")
    kc, vc = dev_u16(case.key_cache), dev_u16(case.value_cache)
    if case.reshape is not None:
        gpu_reshape(case, kc, vc)
    got = gpu_decode(case, kc, vc)
    assert np.array_equal(got, gpu_decode(case, kc, vc)), "not reproducible"
    seqs = None if d.num_seqs <= 8 else sorted(
        {0, d.num_seqs - 1} | set(np.random.default_rng(73).choice(d.num_seqs, 14, replace=False).tolist()))
    okc, ovc = cached_oracle_pools(cfg)
    ref = oracle_decode(case, okc, ovc, seqs=seqs)
    rows = list(range(d.num_seqs)) if seqs is None else seqs
    assert_close(upcast(got)[rows], ref[rows], f"decode (step {step}) cfg{cfg}")
