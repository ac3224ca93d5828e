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
