"""The CPU oracle's row-independent calls spread over host processes — test infrastructure
(used by tests/ and by the benchmark's CPU-baseline leg; never by the library).

The oracle computes every query row of a prefill chunk, and every sequence of a decode batch, on
its own: the row's or sequence's output depends only on its own query and its own keys.  A
full-size case can therefore be cut into parts, each computed by an unchanged oracle call on a
worker process, and the parts put back in order.  Nothing here touches the oracle's arithmetic:
each worker calls the oracle function by name with the `rows` / `seqs` argument the oracle itself
offers, and the parent only concatenates the results.

Workers read the case's arrays from .npy files through read-only memory maps, so a pool of
gigabytes is written once and shared by every process.  They are forked from a forkserver that
`start()` launches before the test process first touches the GPU (tests/conftest.py calls it right
after collection), so no process that holds GPU state is ever forked or replaced.
"""

from __future__ import annotations

import atexit
import concurrent.futures
import multiprocessing
import os
import shutil
import tempfile
from typing import Dict, List, Optional, Sequence

import numpy as np

_CTX = None
_DIR: Optional[str] = None
_POOL: Optional[concurrent.futures.ProcessPoolExecutor] = None
# Host processes the workers may use: the CPU share of the machine, at most 16.
MAX_WORKERS = 16


def workers() -> int:
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(MAX_WORKERS, n))


def start() -> None:
    """Start the forkserver (once).  Call before the process initialises the GPU."""
    global _CTX
    if _CTX is not None:
        return
    ctx = multiprocessing.get_context("forkserver")
    ctx.set_forkserver_preload(["numpy", "oracle.paged_attention"])
    from multiprocessing import forkserver

    # One thread per worker process: the pool itself supplies the parallelism.
    saved = {k: os.environ.get(k) for k in ("OMP_NUM_THREADS", "OPENBLAS_NUM_THREADS", "MKL_NUM_THREADS")}
    for k in saved:
        os.environ[k] = "1"
    try:
        forkserver.ensure_running()
    finally:
        for k, v in saved.items():
            if v is None:
                os.environ.pop(k, None)
            else:
                os.environ[k] = v
    _CTX = ctx


def _pool() -> concurrent.futures.ProcessPoolExecutor:
    global _POOL
    start()
    if _POOL is None:
        _POOL = concurrent.futures.ProcessPoolExecutor(max_workers=workers(), mp_context=_CTX)
        atexit.register(_POOL.shutdown)
    return _POOL


def _scratch_dir() -> str:
    global _DIR
    if _DIR is None:
        _DIR = tempfile.mkdtemp(prefix="pa_oracle_")
        atexit.register(shutil.rmtree, _DIR, True)
    return _DIR


def _call(func_name: str, paths: Dict[str, str], scalars: dict, key: str,
          part: List[int]) -> np.ndarray:
    """Worker: one oracle call over `part` (rows of a chunk, or sequences of a batch)."""
    from oracle import paged_attention as oracle

    arrays = {k: np.load(p, mmap_mode="r") for k, p in paths.items()}
    out = getattr(oracle, func_name)(**arrays, **scalars, **{key: part})
    # The decode functions return the whole batch with only `part` filled; the prefill functions
    # return the requested rows in order.
    return np.asarray(out[part] if key == "seqs" else out)


class Staged:
    """A case's arrays written once to .npy files for the workers; remove() deletes them."""

    def __init__(self, arrays: Dict[str, np.ndarray]):
        self.dir = tempfile.mkdtemp(dir=_scratch_dir())
        self.paths = {}
        for k, a in arrays.items():
            self.paths[k] = os.path.join(self.dir, k + ".npy")
            np.save(self.paths[k], np.ascontiguousarray(a))

    def run(self, func_name: str, scalars: dict, key: str, items: Sequence[int],
            parts: Optional[int] = None) -> np.ndarray:
        """oracle.<func_name>(**arrays, **scalars, <key>=items) computed in parts on the workers,
        the outputs of `items` stacked in the order given."""
        items = [int(i) for i in items]
        if not items:
            return np.zeros((0,))
        n = parts or min(len(items), 2 * workers())
        bounds = np.linspace(0, len(items), n + 1).astype(int)
        chunks = [items[a:b] for a, b in zip(bounds[:-1], bounds[1:]) if b > a]
        futs = [_pool().submit(_call, func_name, self.paths, scalars, key, c) for c in chunks]
        return np.concatenate([f.result() for f in futs], axis=0)

    def remove(self) -> None:
        shutil.rmtree(self.dir, ignore_errors=True)


def warm_up() -> None:
    """Start every worker process (so that a timed run does not include their start-up)."""
    list(_pool().map(_noop, range(4 * workers())))


def _noop(i: int) -> int:
    return i


def run(func_name: str, arrays: Dict[str, np.ndarray], scalars: dict, key: str,
        items: Sequence[int], parts: Optional[int] = None) -> np.ndarray:
    """oracle.<func_name>(**arrays, **scalars, <key>=items), computed in parts on the workers.

    Returns the outputs of `items` stacked in the order given ([len(items)][...]).  `key` is
    "rows" for the prefill functions and "seqs" for the decode functions.
    """
    st = Staged(arrays)
    try:
        return st.run(func_name, scalars, key, items, parts)
    finally:
        st.remove()


def prefill_rows(func_name: str, query, key_cache, value_cache, block_tables, query_start_loc,
                 seq_lens, num_kv_heads, head_dim, block_size, scale, rows=None, **extra):
    """All (or the listed) rows of oracle.prefill_chunk / prefill_chunk_fp8, on the workers."""
    rows = range(np.asarray(query).shape[0]) if rows is None else rows
    arrays = dict(query=query, key_cache=key_cache, value_cache=value_cache,
                  block_tables=block_tables, query_start_loc=query_start_loc, seq_lens=seq_lens)
    scalars = dict(num_kv_heads=int(num_kv_heads), head_dim=int(head_dim),
                   block_size=int(block_size), scale=scale, **extra)
    return run(func_name, arrays, scalars, "rows", rows)


def decode_seqs(func_name: str, query, key_cache, value_cache, block_tables, seq_lens,
                num_kv_heads, head_dim, block_size, scale, seqs=None, **extra):
    """All (or the listed) sequences of oracle.decode / decode_fp8, on the workers, as
    [len(seqs)][Hq][D]."""
    seqs = range(np.asarray(query).shape[0]) if seqs is None else seqs
    arrays = dict(query=query, key_cache=key_cache, value_cache=value_cache,
                  block_tables=block_tables, seq_lens=seq_lens)
    scalars = dict(num_kv_heads=int(num_kv_heads), head_dim=int(head_dim),
                   block_size=int(block_size), scale=scale, **extra)
    return run(func_name, arrays, scalars, "seqs", seqs)
