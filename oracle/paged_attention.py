"""fp64 reference for paged KV-cache attention — test infrastructure, never product code.

The method (PagedAttention as described in the "Serving engine internals" lesson,
section "PagedAttention as a virtual memory system", and the "Inference
optimization" lesson, section "Paged attention") stores the KV cache in
fixed-size physical blocks that may sit anywhere in memory; each sequence reaches
its blocks through a block table that maps logical token positions to physical
block ids.  Paging changes where the bytes live, not what is computed, so this
oracle is the plain definition: scatter new rows into their slots, gather each
sequence's K/V back into logical order through its block table, then run
ordinary max-subtracted softmax attention ("Inference optimization", Build it,
Step 2: attention with a KV cache) in float64.

Physical layout of one (block, KV head) tile, as the library defines it.  A
block of `bs` tokens is split into sub-blocks of 16 tokens.  Within a sub-block
  K is stored as [D/32][16][32]: for each 32-wide slice of the head dimension,
    the 16 tokens' 32 values follow each other;
  V is stored as [D][16]: for each head-dimension index, the 16 tokens' values
    follow each other.
Pools are [num_blocks][num_kv_heads][bs/16][sub-block tile], bf16.
"""

from __future__ import annotations

from typing import Iterable, List, Optional, Sequence, Tuple

import numpy as np

from . import fp8

SUB = 16    # tokens per sub-block
SLICE = 32  # head-dimension slice of the K layout


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact upcast of bf16 bit patterns: bf16 is the top half of an fp32."""
    u = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << np.uint32(16)
    return u.view(np.float32).astype(np.float64)


def _check_shape(num_kv_heads: int, head_dim: int, block_size: int) -> None:
    if block_size % SUB or head_dim % SLICE:
        raise ValueError("block_size must be a multiple of 16 and head_dim of 32")


def _k_view(pool: np.ndarray, Hkv: int, D: int, bs: int) -> np.ndarray:
    """K pool as [N][Hkv][bs/16][D/32][16][32] (a view; no copy)."""
    return pool.reshape(-1, Hkv, bs // SUB, D // SLICE, SUB, SLICE)


def _v_view(pool: np.ndarray, Hkv: int, D: int, bs: int) -> np.ndarray:
    """V pool as [N][Hkv][bs/16][D][16] (a view; no copy)."""
    return pool.reshape(-1, Hkv, bs // SUB, D, SUB)


def logical_blocks_k(pool: np.ndarray, ids: Sequence[int], Hkv: int, D: int, bs: int) -> np.ndarray:
    """K of the given physical blocks as [n][Hkv][bs][D] (token-major), bf16 bits."""
    v = _k_view(pool, Hkv, D, bs)[np.asarray(ids, dtype=np.int64)]
    # [n][Hkv][sb][r][t][c] -> [n][Hkv][sb][t][r][c] -> [n][Hkv][bs][D]
    return v.transpose(0, 1, 2, 4, 3, 5).reshape(len(ids), Hkv, bs, D)


def logical_blocks_v(pool: np.ndarray, ids: Sequence[int], Hkv: int, D: int, bs: int) -> np.ndarray:
    """V of the given physical blocks as [n][Hkv][bs][D] (token-major), bf16 bits."""
    v = _v_view(pool, Hkv, D, bs)[np.asarray(ids, dtype=np.int64)]
    # [n][Hkv][sb][d][t] -> [n][Hkv][sb][t][d] -> [n][Hkv][bs][D]
    return v.transpose(0, 1, 2, 4, 3).reshape(len(ids), Hkv, bs, D)


def reshape_and_cache(key_cache: np.ndarray, value_cache: np.ndarray, key: np.ndarray,
                      value: np.ndarray, slot_mapping: np.ndarray, num_kv_heads: int,
                      head_dim: int, block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """Write each new token's K/V rows into its slot; return the new pool images (copies).

    A slot is `physical block * block_size + offset in block`; the block table
    ("Serving engine internals", PagedAttention section) is what the caller used
    to pick the physical block.  Negative slots are padding and are skipped.
    Slots must be distinct: with two writers for one slot no single result is
    defined, so the oracle refuses such input.
    """
    Hkv, D, bs = num_kv_heads, head_dim, block_size
    _check_shape(Hkv, D, bs)
    slots = np.asarray(slot_mapping, dtype=np.int64)
    live = np.nonzero(slots >= 0)[0]
    s = slots[live]
    n_slots = key_cache.shape[0] * bs
    if s.size and (s.max() >= n_slots):
        raise ValueError("slot beyond the pool")
    if np.unique(s).size != s.size:
        raise ValueError("duplicate slots in one call")
    kc = key_cache.copy()
    vc = value_cache.copy()
    kv = _k_view(kc, Hkv, D, bs)
    vv = _v_view(vc, Hkv, D, bs)
    blk, off = s // bs, s % bs
    sb, t = off // SUB, off % SUB
    k_rows = np.asarray(key)[live].reshape(len(live), Hkv, D // SLICE, SLICE)
    v_rows = np.asarray(value)[live].reshape(len(live), Hkv, D)
    for h in range(Hkv):
        kv[blk, h, sb, :, t, :] = k_rows[:, h]
        vv[blk, h, sb, :, t] = v_rows[:, h]
    return kc, vc


def copy_blocks(key_cache: np.ndarray, value_cache: np.ndarray,
                block_mapping: np.ndarray) -> Tuple[np.ndarray, np.ndarray]:
    """Copy whole physical blocks, K and V, every KV head; return the new pool images (copies).

    Copy-on-write: sequences that share a prompt reference the same physical
    blocks, and a sequence receives its own block only where it diverges from
    the others ("Inference optimization" lesson, Paged attention section;
    vLLM-on-H100 article, PagedAttention section, on rollouts that share a
    prompt's pages until their completions diverge).  A sequence about to write
    into a block that others still reference first gets a fresh block holding a
    copy of the shared one; this is that copy.

    `block_mapping` is int64 [n][2] of (source, destination) block ids.  Each
    destination takes the source's contents as they were before the call.
    Destinations must be distinct and none may also be a source; otherwise the
    result would depend on the order of the copies, so the oracle refuses it.
    """
    m = np.asarray(block_mapping, dtype=np.int64).reshape(-1, 2)
    n = key_cache.shape[0]
    src, dst = m[:, 0], m[:, 1]
    if m.size and (min(src.min(), dst.min()) < 0 or max(src.max(), dst.max()) >= n):
        raise ValueError("block id outside the pool")
    if np.unique(dst).size != dst.size:
        raise ValueError("duplicate destination blocks")
    if np.intersect1d(src, dst).size:
        raise ValueError("a destination block is also a source")
    kc = key_cache.copy()
    vc = value_cache.copy()
    for s, d in zip(src.tolist(), dst.tolist()):
        kc[d] = key_cache[s]
        vc[d] = value_cache[s]
    return kc, vc


def gather_kv(key_cache: np.ndarray, value_cache: np.ndarray, block_table_row: Sequence[int],
              seq_len: int, num_kv_heads: int, head_dim: int,
              block_size: int) -> Tuple[np.ndarray, np.ndarray]:
    """One sequence's K and V in logical order, [seq_len][Hkv][D] float64.

    Logical position p lives in physical block `table[p // bs]` at offset
    `p % bs` ("Serving engine internals", PagedAttention section; "Inference
    optimization", Paged attention section).  Only the first ceil(L/bs) table
    entries are read.
    """
    Hkv, D, bs = num_kv_heads, head_dim, block_size
    _check_shape(Hkv, D, bs)
    nb = -(-int(seq_len) // bs)
    ids = [int(b) for b in block_table_row[:nb]]
    if nb == 0:
        z = np.zeros((0, Hkv, D))
        return z, z.copy()
    k = logical_blocks_k(key_cache, ids, Hkv, D, bs)  # [nb][Hkv][bs][D]
    v = logical_blocks_v(value_cache, ids, Hkv, D, bs)
    k = k.transpose(0, 2, 1, 3).reshape(nb * bs, Hkv, D)[:seq_len]
    v = v.transpose(0, 2, 1, 3).reshape(nb * bs, Hkv, D)[:seq_len]
    return bf16_to_f64(k), bf16_to_f64(v)


def attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: float,
              rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Attention of Tq query rows over L cached keys, float64.

    q [Tq][Hq][D], k/v [L][Hkv][D].  Query head h reads KV head h // (Hq/Hkv):
    consecutive query heads share a KV head (grouped-query attention, "Inference
    optimization" exercises).  The query rows are the last Tq positions of the
    sequence, so row i may attend to keys 0 .. L-Tq+i: the causal mask of Step 2
    with its diagonal offset `seq_len_k - seq_len_q + 1`.  Keys outside the mask
    are excluded outright, which equals adding a large negative number before
    the exponential.  Softmax subtracts the row maximum before exponentiating.
    `rows` restricts the computation to some query rows (for large cases).
    """
    Tq, Hq, D = q.shape
    L, Hkv, _ = k.shape
    G = Hq // Hkv
    if rows is None:
        rows = range(Tq)
    rows = np.asarray(list(rows), dtype=np.int64)
    out = np.zeros((len(rows), Hq, D))
    if L == 0:
        return out  # softmax over no keys: defined as a zero output
    limit = L - Tq + rows  # last visible key per selected row
    visible = np.arange(L)[None, :] <= limit[:, None]  # [R][L]
    for h in range(Hkv):
        qg = q[rows, h * G:(h + 1) * G, :]                      # [R][G][D]
        s = np.einsum("rgd,ld->rgl", qg, k[:, h, :]) * float(scale)
        s = np.where(visible[:, None, :], s, -np.inf)
        m = s.max(axis=-1, keepdims=True)
        w = np.exp(s - m)
        w = np.where(visible[:, None, :], w, 0.0)
        num = np.einsum("rgl,ld->rgd", w, v[:, h, :])
        out[:, h * G:(h + 1) * G, :] = num / w.sum(axis=-1, keepdims=True)
    return out


def decode(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
           block_tables: np.ndarray, seq_lens: np.ndarray, num_kv_heads: int, head_dim: int,
           block_size: int, scale: float, seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """Decode: one query token per sequence against its whole cached context.

    query is bf16 bits [B][Hq][D]; returns [B][Hq][D] float64 (rows of sequences
    not in `seqs` are left zero).  A sequence of length 0 yields zeros.
    """
    B, Hq, D = query.shape
    out = np.zeros((B, Hq, D))
    for s in (range(B) if seqs is None else seqs):
        k, v = gather_kv(key_cache, value_cache, block_tables[s], int(seq_lens[s]),
                         num_kv_heads, head_dim, block_size)
        q = bf16_to_f64(query[s])[None]
        out[s] = attention(q, k, v, scale)[0]
    return out


def prefill_chunk(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                  block_tables: np.ndarray, query_start_loc: np.ndarray, seq_lens: np.ndarray,
                  num_kv_heads: int, head_dim: int, block_size: int, scale: float,
                  rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Chunked prefill: each sequence's chunk of query rows, causally, over its paged context.

    Chunk i holds query rows query_start_loc[i] .. query_start_loc[i+1]-1, which
    are the last positions of a sequence of seq_lens[i] cached tokens (its own
    K/V already written).  Chunked prefill is described in the "Serving engine
    internals" lesson (chunked-prefill section): a long prompt is processed as
    fixed-size slices that attend to everything cached before them.
    Returns [total_q][Hq][D] float64, or only the rows listed in `rows`
    (global row indices) in that order.
    """
    total_q, Hq, D = query.shape
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    want = np.arange(total_q) if rows is None else np.asarray(list(rows), dtype=np.int64)
    out = np.zeros((len(want), Hq, D))
    for i in range(len(qsl) - 1):
        lo, hi = int(qsl[i]), int(qsl[i + 1])
        sel = np.nonzero((want >= lo) & (want < hi))[0]
        if sel.size == 0:
            continue
        k, v = gather_kv(key_cache, value_cache, block_tables[i], int(seq_lens[i]),
                         num_kv_heads, head_dim, block_size)
        q = bf16_to_f64(query[lo:hi])
        out[sel] = attention(q, k, v, scale, rows=(want[sel] - lo).tolist())
    return out


def contiguous_attention(q: np.ndarray, k_contig: np.ndarray, v_contig: np.ndarray,
                         scale: float) -> np.ndarray:
    """Attention over an unpaged cache, as the Step 1 KVCache of the "Inference
    optimization" lesson keeps it: one array per sequence with positions in order."""
    return attention(q, k_contig, v_contig, scale)


# ------------------------------------------------------------------------------------------
# FP8 (E4M3) KV cache: the same block layout with one-byte codes, one scale per pool.
# ------------------------------------------------------------------------------------------

def reshape_and_cache_fp8(key_cache: np.ndarray, value_cache: np.ndarray, key: np.ndarray,
                          value: np.ndarray, slot_mapping: np.ndarray, num_kv_heads: int,
                          head_dim: int, block_size: int, k_scale: float,
                          v_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """Quantise each new token's bf16 K/V rows to E4M3 codes (code = encode(x / scale), see
    oracle.fp8) and write them into their slots of uint8 pools laid out like the bf16 pools,
    one byte per element.  Returns the new pool images (copies)."""
    return reshape_and_cache(key_cache, value_cache, fp8.quantize(key, k_scale),
                             fp8.quantize(value, v_scale), slot_mapping, num_kv_heads, head_dim,
                             block_size)


def gather_kv_fp8(key_cache: np.ndarray, value_cache: np.ndarray, block_table_row: Sequence[int],
                  seq_len: int, num_kv_heads: int, head_dim: int, block_size: int, k_scale: float,
                  v_scale: float) -> Tuple[np.ndarray, np.ndarray]:
    """One sequence's dequantised K and V in logical order, [seq_len][Hkv][D] float64:
    scale * value of the code, through the block table exactly as gather_kv."""
    Hkv, D, bs = num_kv_heads, head_dim, block_size
    _check_shape(Hkv, D, bs)
    nb = -(-int(seq_len) // bs)
    if nb == 0:
        z = np.zeros((0, Hkv, D))
        return z, z.copy()
    ids = [int(b) for b in block_table_row[:nb]]
    k = logical_blocks_k(key_cache, ids, Hkv, D, bs)
    v = logical_blocks_v(value_cache, ids, Hkv, D, bs)
    k = k.transpose(0, 2, 1, 3).reshape(nb * bs, Hkv, D)[:seq_len]
    v = v.transpose(0, 2, 1, 3).reshape(nb * bs, Hkv, D)[:seq_len]
    return float(k_scale) * fp8.decode(k), float(v_scale) * fp8.decode(v)


def decode_fp8(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
               block_tables: np.ndarray, seq_lens: np.ndarray, num_kv_heads: int, head_dim: int,
               block_size: int, scale: float, k_scale: float, v_scale: float,
               seqs: Optional[Iterable[int]] = None) -> np.ndarray:
    """Decode over an FP8 cache: the attention of `decode` on the dequantised keys and values."""
    B, Hq, D = query.shape
    out = np.zeros((B, Hq, D))
    for s in (range(B) if seqs is None else seqs):
        k, v = gather_kv_fp8(key_cache, value_cache, block_tables[s], int(seq_lens[s]),
                             num_kv_heads, head_dim, block_size, k_scale, v_scale)
        out[s] = attention(bf16_to_f64(query[s])[None], k, v, scale)[0]
    return out


def prefill_chunk_fp8(query: np.ndarray, key_cache: np.ndarray, value_cache: np.ndarray,
                      block_tables: np.ndarray, query_start_loc: np.ndarray, seq_lens: np.ndarray,
                      num_kv_heads: int, head_dim: int, block_size: int, scale: float,
                      k_scale: float, v_scale: float,
                      rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """Chunked prefill over an FP8 cache: the attention of `prefill_chunk` on the dequantised
    keys and values."""
    total_q, Hq, D = query.shape
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    want = np.arange(total_q) if rows is None else np.asarray(list(rows), dtype=np.int64)
    out = np.zeros((len(want), Hq, D))
    for i in range(len(qsl) - 1):
        lo, hi = int(qsl[i]), int(qsl[i + 1])
        sel = np.nonzero((want >= lo) & (want < hi))[0]
        if sel.size == 0:
            continue
        k, v = gather_kv_fp8(key_cache, value_cache, block_tables[i], int(seq_lens[i]),
                             num_kv_heads, head_dim, block_size, k_scale, v_scale)
        out[sel] = attention(bf16_to_f64(query[lo:hi]), k, v, scale, rows=(want[sel] - lo).tolist())
    return out
