"""Seeded input generation for the five paged-attention workloads and for small test cases.

Workload shapes follow the pages: block size 16 by default ("Serving engine
internals" lesson, PagedAttention section; the vLLM-on-H100 article says 16 or
32), Llama-3-70B-like GQA with 64 query / 8 KV heads and head_dim 128
("Inference optimization" lesson, KV cache section and exercises), concurrency
128 and a mean of 1,500 tokens against an 8,192-token reservation ("Serving
engine internals", PagedAttention section and exercise 4, which also gives the
600-token standard deviation), 32k prompts cut into 512-token chunks (same
lesson, chunked-prefill section), 8 or 16 rollouts sharing one prompt's pages
(vLLM-on-H100 article, PagedAttention section) and a 16-layer, 4-KV-head,
head_dim-256 model at 8,192 tokens (same article, first section).

Nothing here computes attention.  Slot numbers are the caller-side addressing
a scheduler performs (block id times block size plus the offset in the block).
"""

from __future__ import annotations

import concurrent.futures
import dataclasses
import math
import os
import threading
from typing import Dict, List, Optional, Sequence, Tuple

import numpy as np

BF16_NAN = np.uint16(0x7FC0)

# Normal draws for large arrays are made in fixed chunks of this many values.  Chunk c of a draw
# uses its own generator seeded with (case seed, draw label, c), so chunks are independent and can
# be filled by several threads; the result does not depend on the thread count.
_CHUNK = 1 << 22
_THREADS = max(1, min(16, len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else 4))


def bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even); return the bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    out = np.empty(x.shape, dtype=np.uint16)
    _bf16_into(x.reshape(-1), out.reshape(-1), np.empty(x.size, dtype=np.uint32))
    return out


def _bf16_into(x: np.ndarray, out: np.ndarray, tmp: np.ndarray) -> None:
    """bf16 rounding of float32 `x` into uint16 `out`, using uint32 scratch `tmp` (same length)."""
    u = x.view(np.uint32)
    np.right_shift(u, 16, out=tmp)
    np.bitwise_and(tmp, 1, out=tmp)
    np.add(tmp, 0x7FFF, out=tmp)
    np.add(tmp, u, out=tmp)
    np.right_shift(tmp, 16, out=tmp)
    out[...] = tmp
    nan = np.isnan(x)
    if nan.any():
        out[nan] = BF16_NAN


def normal_bf16(seed: Sequence[int], label: int, count: int) -> np.ndarray:
    """`count` N(0,1) draws rounded to bf16, as a flat uint16 array (see _CHUNK)."""
    out = np.empty(count, dtype=np.uint16)
    starts = list(range(0, count, _CHUNK))
    local = threading.local()

    def fill(ci: int) -> None:
        if not hasattr(local, "f"):
            local.f = np.empty(_CHUNK, dtype=np.float32)
            local.u = np.empty(_CHUNK, dtype=np.uint32)
        start = starts[ci]
        n = min(_CHUNK, count - start)
        g = np.random.default_rng([*seed, label, ci])
        f = local.f[:n]
        g.standard_normal(out=f, dtype=np.float32)
        _bf16_into(f, out[start:start + n], local.u[:n])

    if len(starts) <= 1:
        for ci in range(len(starts)):
            fill(ci)
    else:
        with concurrent.futures.ThreadPoolExecutor(max_workers=min(_THREADS, len(starts))) as ex:
            list(ex.map(fill, range(len(starts))))
    return out


def lognormal_lengths(rng: np.random.Generator, n: int, mean: float = 1500.0, std: float = 600.0,
                      lo: int = 16, hi: int = 8192) -> np.ndarray:
    """Context lengths: lognormal with the given mean and standard deviation, rounded, clipped."""
    sigma = math.sqrt(math.log1p((std / mean) ** 2))
    mu = math.log(mean) - 0.5 * sigma * sigma
    x = rng.lognormal(mu, sigma, size=n)
    return np.clip(np.rint(x), lo, hi).astype(np.int64)


class BlockAllocator:
    """Free list of physical block ids with reference counts (host side).

    Blocks are handed out from a shuffled free list, so a sequence's blocks land
    anywhere in the pool.  A block shared by several sequences (a common prompt)
    carries one reference per holder and returns to the free list only when the
    last holder releases it.
    """

    def __init__(self, num_blocks: int, rng: Optional[np.random.Generator] = None):
        ids = np.arange(num_blocks, dtype=np.int64)
        if rng is not None:
            ids = rng.permutation(ids)
        self._free: List[int] = [int(i) for i in ids[::-1]]  # pop() from the end
        self._ref = np.zeros(num_blocks, dtype=np.int64)
        self.num_blocks = num_blocks

    @property
    def num_free(self) -> int:
        return len(self._free)

    def can_allocate(self, n: int) -> bool:
        return n <= len(self._free)

    def allocate(self, n: int) -> List[int]:
        if n > len(self._free):
            raise MemoryError(f"block pool exhausted: want {n}, have {len(self._free)} free")
        out = [self._free.pop() for _ in range(n)]
        for b in out:
            self._ref[b] = 1
        return out

    def share(self, ids: Sequence[int]) -> None:
        for b in ids:
            if self._ref[b] <= 0:
                raise ValueError(f"cannot share block {b}: not allocated")
            self._ref[b] += 1

    def release(self, ids: Sequence[int]) -> None:
        for b in ids:
            if self._ref[b] <= 0:
                raise ValueError(f"double free of block {b}")
            self._ref[b] -= 1
            if self._ref[b] == 0:
                self._free.append(int(b))

    def refcount(self, b: int) -> int:
        return int(self._ref[b])

    def prepare_write(self, table: List[int], pos: int, block_size: int) -> Optional[Tuple[int, int]]:
        """Copy-on-write before a sequence writes logical position `pos`.

        If the block holding `pos` is still referenced by other sequences, the
        writer takes a fresh block, drops its reference to the shared one and
        points its table entry at the fresh block; the returned (source,
        destination) pair is the copy that must run before the write.  A block
        with a single holder is written in place (returns None), so the last
        sequence still holding a shared block keeps it.
        """
        j = pos // block_size
        b = int(table[j])
        if self._ref[b] <= 1:
            return None
        fresh = self.allocate(1)[0]
        self.release([b])
        table[j] = fresh
        return b, fresh


@dataclasses.dataclass
class DecodeBatch:
    block_tables: np.ndarray  # int32 [B][max_blocks]; padding entries hold the poison block
    seq_lens: np.ndarray      # int32 [B]; cached tokens including the one being decoded
    query: np.ndarray         # uint16 (bf16 bits) [B][Hq][D]

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.seq_lens.size else 0


@dataclasses.dataclass
class PrefillBatch:
    block_tables: np.ndarray     # int32 [n][max_blocks]
    seq_lens: np.ndarray         # int32 [n]; prior context plus the chunk
    query_start_loc: np.ndarray  # int32 [n+1]; chunk i's rows are query[qsl[i]:qsl[i+1]]
    query: np.ndarray            # uint16 [total_q][Hq][D]

    @property
    def num_seqs(self) -> int:
        return int(self.seq_lens.shape[0])

    @property
    def total_q(self) -> int:
        return int(self.query_start_loc[-1])

    @property
    def max_q_len(self) -> int:
        return int(np.diff(self.query_start_loc).max()) if self.num_seqs else 0

    @property
    def max_seq_len(self) -> int:
        return int(self.seq_lens.max()) if self.num_seqs else 0


@dataclasses.dataclass
class ReshapeBatch:
    key: np.ndarray           # uint16 [T][Hkv][D]
    value: np.ndarray         # uint16 [T][Hkv][D]
    slot_mapping: np.ndarray  # int64 [T]; block id * block_size + offset, negative = skip


@dataclasses.dataclass
class Case:
    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    num_blocks: int               # including the poison block
    poison_block: int
    scale: np.float32
    key_cache: np.ndarray         # uint16 [num_blocks][Hkv*block_size*head_dim]
    value_cache: np.ndarray       # uint16 [num_blocks][Hkv*block_size*head_dim]
    reshape: Optional[ReshapeBatch] = None
    decode: Optional[DecodeBatch] = None
    prefill: Optional[PrefillBatch] = None
    info: Dict[str, object] = dataclasses.field(default_factory=dict)

    @property
    def block_elems(self) -> int:
        return self.num_kv_heads * self.block_size * self.head_dim


@dataclasses.dataclass
class Spec:
    """What to generate.  Lengths are final cached lengths (including new tokens)."""

    name: str
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int
    seed: Tuple[int, ...]
    decode_lens: Sequence[int] = ()
    prefill: Sequence[Tuple[int, int]] = ()   # (prior context, chunk length) per chunk sequence
    decode_new_token: bool = False            # reshape one new token per decode sequence (at position L-1)
    prefill_new_tokens: bool = False          # reshape the chunk's own tokens before attention
    share_groups: Sequence[Tuple[Sequence[int], int]] = ()  # (decode seq indices, shared prefix tokens)
    pool_blocks: Optional[int] = None         # usable blocks; default ceil(pool_slack * needed)
    pool_slack: float = 1.1


def _blocks_for(n_tokens: int, bs: int) -> int:
    return -(-n_tokens // bs)


def build_case(spec: Spec) -> Case:
    """Generate one workload.  Block ids come from one generator seeded with the spec's seed;
    queries, K pool, V pool and new K/V rows are separate labelled normal draws (labels 1..6)."""
    rng = np.random.default_rng(list(spec.seed))
    Hq, Hkv, D, bs = spec.num_q_heads, spec.num_kv_heads, spec.head_dim, spec.block_size
    dec_lens = [int(x) for x in spec.decode_lens]
    pre = [(int(c), int(q)) for c, q in spec.prefill]

    # --- block accounting -------------------------------------------------------------
    shared_of: Dict[int, Tuple[int, int]] = {}  # decode seq -> (group id, shared blocks)
    for gid, (members, shared_tokens) in enumerate(spec.share_groups):
        if shared_tokens % bs:
            raise ValueError("shared prefixes must cover whole blocks")
        for m in members:
            shared_of[int(m)] = (gid, shared_tokens // bs)
    needed = sum(_blocks_for(c + q, bs) for c, q in pre)
    group_blocks = {gid: sh // bs for gid, (_, sh) in enumerate(spec.share_groups)}
    needed += sum(group_blocks.values())
    for i, L in enumerate(dec_lens):
        nb = _blocks_for(L, bs)
        if i in shared_of:
            gid, sb = shared_of[i]
            if nb < sb:
                raise ValueError("sequence shorter than its shared prefix")
            nb -= sb
        needed += nb
    usable = spec.pool_blocks if spec.pool_blocks is not None else math.ceil(spec.pool_slack * needed)
    if usable < needed:
        raise ValueError(f"pool of {usable} blocks cannot hold {needed}")
    num_blocks = usable + 1
    poison = usable  # the extra last block: NaN-filled, used for table padding
    alloc = BlockAllocator(usable, rng)

    pre_tables: List[List[int]] = [alloc.allocate(_blocks_for(c + q, bs)) for c, q in pre]
    group_ids = {gid: alloc.allocate(n) for gid, n in group_blocks.items()}
    dec_tables: List[List[int]] = []
    for i, L in enumerate(dec_lens):
        nb = _blocks_for(L, bs)
        if i in shared_of:
            gid, sb = shared_of[i]
            alloc.share(group_ids[gid])
            dec_tables.append(list(group_ids[gid]) + alloc.allocate(nb - sb))
        else:
            dec_tables.append(alloc.allocate(nb))

    def pad(tables: List[List[int]]) -> np.ndarray:
        width = max([len(t) for t in tables] + [1])
        out = np.full((len(tables), width), poison, dtype=np.int32)
        for r, t in enumerate(tables):
            out[r, :len(t)] = t
        return out

    # --- draws ----------------------------------------------------------------------
    n_dec = len(dec_lens)
    total_q = sum(q for _, q in pre)
    seed = tuple(spec.seed)
    q_dec = normal_bf16(seed, 1, n_dec * Hq * D).reshape(n_dec, Hq, D)
    q_pre = normal_bf16(seed, 2, total_q * Hq * D).reshape(total_q, Hq, D)
    elems = Hkv * bs * D
    kc = normal_bf16(seed, 3, num_blocks * elems).reshape(num_blocks, elems)
    vc = normal_bf16(seed, 4, num_blocks * elems).reshape(num_blocks, elems)
    kc[poison] = BF16_NAN
    vc[poison] = BF16_NAN

    # --- new tokens to scatter ------------------------------------------------------
    slots: List[int] = []
    if spec.prefill_new_tokens:
        for (c, q), t in zip(pre, pre_tables):
            for p in range(c, c + q):
                slots.append(t[p // bs] * bs + p % bs)
    if spec.decode_new_token:
        for L, t in zip(dec_lens, dec_tables):
            p = L - 1
            slots.append(t[p // bs] * bs + p % bs)
    reshape = None
    if slots:
        T = len(slots)
        reshape = ReshapeBatch(
            key=normal_bf16(seed, 5, T * Hkv * D).reshape(T, Hkv, D),
            value=normal_bf16(seed, 6, T * Hkv * D).reshape(T, Hkv, D),
            slot_mapping=np.asarray(slots, dtype=np.int64),
        )

    decode = None
    if n_dec:
        decode = DecodeBatch(block_tables=pad(dec_tables),
                             seq_lens=np.asarray(dec_lens, dtype=np.int32), query=q_dec)
    prefill = None
    if pre:
        qsl = np.zeros(len(pre) + 1, dtype=np.int32)
        qsl[1:] = np.cumsum([q for _, q in pre])
        prefill = PrefillBatch(block_tables=pad(pre_tables),
                               seq_lens=np.asarray([c + q for c, q in pre], dtype=np.int32),
                               query_start_loc=qsl, query=q_pre)
    info = {"pool_blocks_usable": usable, "blocks_needed": needed,
            "decode_lens": dec_lens, "prefill": pre}
    return Case(name=spec.name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                num_blocks=num_blocks, poison_block=poison,
                scale=np.float32(1.0 / math.sqrt(D)), key_cache=kc, value_cache=vc,
                reshape=reshape, decode=decode, prefill=prefill, info=info)


def build_cow_case(name: str, num_prompts: int, candidates: int, prompt_len: int,
                   num_q_heads: int, num_kv_heads: int, head_dim: int, block_size: int,
                   seed: Tuple[int, ...], tails: Optional[Sequence[int]] = None,
                   pool_slack: float = 1.1) -> Tuple[Case, np.ndarray]:
    """Rollouts that share a prompt whose last block is only partly filled, at the step where
    each candidate writes its next token.

    Every candidate of a group references the prompt's blocks, the last one partial (prompt_len
    need not be a multiple of block_size).  Candidate c already holds `tails[c]` generated tokens
    (default 0); the first tokens of a tail that fall into the shared partial block were written
    into a private copy of it when that candidate diverged.  The step appends one token per
    candidate at position prompt_len + tail; a candidate whose token lands in a block still
    shared gets a copy first (BlockAllocator.prepare_write).  Returns the case, whose reshape
    batch holds the new tokens and whose decode batch attends prompt_len + tail + 1 keys, and the
    int64 [n][2] (source, destination) copies to run before the reshape.  The pool holds the
    state before the step: drawn contents everywhere, the private copies already made.
    """
    rng = np.random.default_rng(list(seed))
    Hq, Hkv, D, bs = num_q_heads, num_kv_heads, head_dim, block_size
    B = num_prompts * candidates
    tails = [0] * B if tails is None else [int(t) for t in tails]
    shared_blocks = _blocks_for(prompt_len, bs)
    lens = [prompt_len + t + 1 for t in tails]
    # Upper bound of the blocks the step can need: the shared prompt blocks once per group, each
    # candidate's private blocks, and one copy per candidate.
    needed = num_prompts * shared_blocks + sum(_blocks_for(L, bs) for L in lens) + B
    usable = math.ceil(pool_slack * needed)
    num_blocks = usable + 1
    poison = usable
    alloc = BlockAllocator(usable, rng)

    elems = Hkv * bs * D
    kc = normal_bf16(seed, 3, num_blocks * elems).reshape(num_blocks, elems)
    vc = normal_bf16(seed, 4, num_blocks * elems).reshape(num_blocks, elems)
    kc[poison] = BF16_NAN
    vc[poison] = BF16_NAN

    tables: List[List[int]] = []
    for g in range(num_prompts):
        prompt = alloc.allocate(shared_blocks)
        alloc.share(prompt * (candidates - 1))
        for c in range(candidates):
            t = list(prompt)
            tail = tails[g * candidates + c]
            # Earlier divergence: a tail that reached into the partial block made a private copy.
            if tail > 0 and prompt_len % bs:
                pair = alloc.prepare_write(t, prompt_len, bs)
                if pair is not None:
                    kc[pair[1]] = kc[pair[0]]
                    vc[pair[1]] = vc[pair[0]]
            extra = _blocks_for(prompt_len + tail, bs) - shared_blocks
            if extra > 0:
                t += alloc.allocate(extra)
            tables.append(t)

    tables_before = [list(t) for t in tables]
    # The step: one new token per candidate at position prompt_len + tail.
    copies: List[Tuple[int, int]] = []
    slots: List[int] = []
    for b, t in enumerate(tables):
        pos = prompt_len + tails[b]
        if pos // bs >= len(t):
            t += alloc.allocate(1)
        pair = alloc.prepare_write(t, pos, bs)
        if pair is not None:
            copies.append(pair)
        slots.append(t[pos // bs] * bs + pos % bs)

    width = max(len(t) for t in tables)
    bt = np.full((B, width), poison, dtype=np.int32)
    for r, t in enumerate(tables):
        bt[r, :len(t)] = t
    reshape = ReshapeBatch(key=normal_bf16(seed, 5, B * Hkv * D).reshape(B, Hkv, D),
                           value=normal_bf16(seed, 6, B * Hkv * D).reshape(B, Hkv, D),
                           slot_mapping=np.asarray(slots, dtype=np.int64))
    decode = DecodeBatch(block_tables=bt, seq_lens=np.asarray(lens, dtype=np.int32),
                         query=normal_bf16(seed, 1, B * Hq * D).reshape(B, Hq, D))
    info = {"pool_blocks_usable": usable, "prompt_len": prompt_len, "tails": tails,
            "copies": len(copies), "free_blocks_after": alloc.num_free,
            "tables_before": tables_before}
    case = Case(name=name, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                num_blocks=num_blocks, poison_block=poison, scale=np.float32(1.0 / math.sqrt(D)),
                key_cache=kc, value_cache=vc, reshape=reshape, decode=decode, info=info)
    return case, np.asarray(copies, dtype=np.int64).reshape(-1, 2)


# ----------------------------------------------------------------------------------------
# The five named workloads.
# ----------------------------------------------------------------------------------------

def _spec_tiny() -> Spec:
    # Four requests of 50, 120, 240 and 1,024 tokens (vLLM-on-H100 article, continuous
    # batching section); each gets one new token written at position L0, so it attends L0+1 keys.
    lens0 = [50, 120, 240, 1024]
    return Spec(name="tiny_decode", num_q_heads=8, num_kv_heads=2, head_dim=64, block_size=16,
                seed=(444, 1), decode_lens=[x + 1 for x in lens0], decode_new_token=True,
                pool_blocks=128)


def _spec_llama70b_decode(batch: int = 128, seed_id: int = 2) -> Spec:
    rng = np.random.default_rng([444, seed_id, 0])
    lens = lognormal_lengths(rng, batch)
    return Spec(name="llama70b_decode_b128", num_q_heads=64, num_kv_heads=8, head_dim=128,
                block_size=16, seed=(444, seed_id), decode_lens=lens.tolist())


def _spec_widehead() -> Spec:
    return Spec(name="widehead_decode_b64_8k", num_q_heads=16, num_kv_heads=4, head_dim=256,
                block_size=32, seed=(444, 3), decode_lens=[8192] * 64, pool_blocks=64 * 256)


def _spec_mixed() -> Spec:
    rng = np.random.default_rng([444, 4, 0])
    lens = lognormal_lengths(rng, 127)
    return Spec(name="mixed_prefill512_ctx31744_plus_decode127", num_q_heads=64, num_kv_heads=8,
                head_dim=128, block_size=16, seed=(444, 4), decode_lens=lens.tolist(),
                prefill=[(31744, 512)], prefill_new_tokens=True)


def _spec_prefix_shared() -> Spec:
    rng = np.random.default_rng([444, 5, 0])
    tails = rng.integers(0, 1025, size=128)
    lens = [4096 + int(t) + 1 for t in tails]
    groups = [(list(range(16 * g, 16 * g + 16)), 4096) for g in range(8)]
    return Spec(name="prefix_shared_8x16_prompt4096", num_q_heads=64, num_kv_heads=8, head_dim=128,
                block_size=16, seed=(444, 5), decode_lens=lens, decode_new_token=True,
                share_groups=groups)


def _spec_tp_share(tp: int = 8) -> Spec:
    # One GPU's share of the Llama-3.3-70B-shaped decode when its 8 KV heads are split over `tp`
    # GPUs: the same 128 sequences and lengths as the batch-128 workload, with 8/tp KV heads and
    # their 64/tp query heads.
    rng = np.random.default_rng([444, 2, 0])
    lens = lognormal_lengths(rng, 128)
    return Spec(name=f"llama70b_decode_b128_tp{tp}_share", num_q_heads=64 // tp,
                num_kv_heads=8 // tp, head_dim=128, block_size=16, seed=(444, 2, tp),
                decode_lens=lens.tolist())


def tp_share_case(tp: int = 8) -> Case:
    """The 70B-shaped batch-128 decode as one GPU's share under tensor parallelism over KV heads
    (tp divides 8): Hq = 64/tp, Hkv = 8/tp, same lengths."""
    if tp not in (1, 2, 4, 8):
        raise ValueError("tp must divide the 8 KV heads")
    return build_case(_spec_tp_share(tp))


NAMED_CASES = {
    1: _spec_tiny,
    2: _spec_llama70b_decode,
    3: _spec_widehead,
    4: _spec_mixed,
    5: _spec_prefix_shared,
}


def named_case(cfg_id: int) -> Case:
    """Build workload `cfg_id` (1..5) at full size."""
    return build_case(NAMED_CASES[cfg_id]())
