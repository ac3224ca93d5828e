"""Glue between the seeded workloads, the CPU oracle and the HIP library for the tests."""

from __future__ import annotations

import functools

import numpy as np
import torch

from oracle import paged_attention as oracle
from workloads import Case, named_case

ATOL = 1e-2
RTOL = 1e-2


def has_gpu() -> bool:
    return torch.cuda.is_available()


def dev_u16(a: np.ndarray) -> torch.Tensor:
    """bf16 bit patterns (uint16) -> GPU bfloat16 tensor with the same bits."""
    return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)


def host_u16(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def dev_i32(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).cuda()


def dev_i64(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).cuda()


def upcast(t_u16: np.ndarray) -> np.ndarray:
    return oracle.bf16_to_f64(t_u16)


def tol_ratio(gpu: np.ndarray, ref: np.ndarray) -> float:
    """max |gpu - ref| / (atol + rtol*|ref|); <= 1 passes."""
    if gpu.size == 0:
        return 0.0
    r = np.abs(gpu - ref) / (ATOL + RTOL * np.abs(ref))
    r = np.where(np.isnan(r), np.inf, r)
    return float(r.max())


def assert_close(gpu: np.ndarray, ref: np.ndarray, what: str) -> None:
    ratio = tol_ratio(gpu, ref)
    assert ratio <= 1.0, f"{what}: max error ratio {ratio:.3f} (|gpu-oracle| <= 1e-2 + 1e-2*|oracle|)"


def oracle_pools_after_reshape(case: Case):
    """Pool images after the case's reshape step, as the oracle computes them."""
    if case.reshape is None:
        return case.key_cache, case.value_cache
    r = case.reshape
    return oracle.reshape_and_cache(case.key_cache, case.value_cache, r.key, r.value, r.slot_mapping,
                                    case.num_kv_heads, case.head_dim, case.block_size)


@functools.lru_cache(maxsize=2)
def cached_named_case(cfg_id: int) -> Case:
    return named_case(cfg_id)


@functools.lru_cache(maxsize=2)
def cached_oracle_pools(cfg_id: int):
    return oracle_pools_after_reshape(cached_named_case(cfg_id))


def oracle_quantize_pool(pool_u16: np.ndarray, scale: float) -> np.ndarray:
    """E4M3 codes of a whole bf16 pool by the oracle's quantiser, in chunks on several threads
    (the result is the same as one call over the whole array)."""
    import concurrent.futures
    import os

    from oracle import fp8

    flat = np.ascontiguousarray(pool_u16).reshape(-1)
    out = np.empty(flat.shape, dtype=np.uint8)
    step = 1 << 23
    starts = list(range(0, flat.size, step))

    def work(a):
        out[a:a + step] = fp8.quantize(flat[a:a + step], scale)

    threads = max(1, min(16, len(os.sched_getaffinity(0))))
    with concurrent.futures.ThreadPoolExecutor(max_workers=threads) as ex:
        list(ex.map(work, starts))
    return out.reshape(pool_u16.shape)


def dev_u8(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def host_u8(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy()


# Per-tensor FP8 scales for the N(0,1) workloads: the largest of ~10^8 normal draws (about 6)
# maps near the E4M3 maximum 448.
FP8_K_SCALE = 6.0 / 448.0
FP8_V_SCALE = 5.5 / 448.0


@functools.lru_cache(maxsize=2)
def cached_fp8_pools(cfg_id: int):
    """E4M3 pools of a named workload: its bf16 pools after the step's reshape (the oracle's),
    quantised whole by the oracle's quantiser with FP8_K_SCALE / FP8_V_SCALE."""
    okc, ovc = cached_oracle_pools(cfg_id)
    return oracle_quantize_pool(okc, FP8_K_SCALE), oracle_quantize_pool(ovc, FP8_V_SCALE)


@functools.lru_cache(maxsize=16)
def full_decode_oracle(cfg_id: int, fp8: bool = False) -> np.ndarray:
    """Oracle decode of every sequence of a named workload ([B][Hq][D] float64), over the pools
    after the step's reshape (bf16, or their E4M3 codes), computed on several host processes."""
    from oracle import pool as oracle_pool

    case = cached_named_case(cfg_id)
    d = case.decode
    kc, vc = cached_fp8_pools(cfg_id) if fp8 else cached_oracle_pools(cfg_id)
    extra = dict(k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE) if fp8 else {}
    return oracle_pool.decode_seqs("decode_fp8" if fp8 else "decode", d.query, kc, vc,
                                   d.block_tables, d.seq_lens, case.num_kv_heads, case.head_dim,
                                   case.block_size, case.scale, **extra)


@functools.lru_cache(maxsize=2)
def full_prefill_oracle(cfg_id: int, fp8: bool = False) -> np.ndarray:
    """Oracle output of every query row of a named workload's prefill chunk ([total_q][Hq][D]
    float64), over the pools after the chunk's reshape (bf16, or their E4M3 codes), computed on
    several host processes."""
    from oracle import pool as oracle_pool

    case = cached_named_case(cfg_id)
    p = case.prefill
    kc, vc = cached_fp8_pools(cfg_id) if fp8 else cached_oracle_pools(cfg_id)
    extra = dict(k_scale=FP8_K_SCALE, v_scale=FP8_V_SCALE) if fp8 else {}
    return oracle_pool.prefill_rows("prefill_chunk_fp8" if fp8 else "prefill_chunk", p.query, kc,
                                    vc, p.block_tables, p.query_start_loc, p.seq_lens,
                                    case.num_kv_heads, case.head_dim, case.block_size, case.scale,
                                    **extra)


@functools.lru_cache(maxsize=1)
def cached_tp_share_case(tp: int = 8) -> Case:
    from workloads import tp_share_case

    return tp_share_case(tp)


@functools.lru_cache(maxsize=1)
def full_tp_share_oracle(tp: int = 8) -> np.ndarray:
    """Oracle decode of every sequence of the 70B-shaped batch's tensor-parallel share."""
    from oracle import pool as oracle_pool

    case = cached_tp_share_case(tp)
    d = case.decode
    return oracle_pool.decode_seqs("decode", d.query, case.key_cache, case.value_cache,
                                   d.block_tables, d.seq_lens, case.num_kv_heads, case.head_dim,
                                   case.block_size, case.scale)
