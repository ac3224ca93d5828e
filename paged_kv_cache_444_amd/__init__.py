"""Python binding of libpagedattn (paged KV-cache attention for MI355X / gfx950).

Argument marshalling only: every operation runs in the library's HIP kernels.  Tensors are torch
tensors on the current HIP device; their data pointers and torch's current stream are handed to the
C ABI declared in include/pa.h.  There is no fallback: if the shared library is missing or fails to
load, importing the ops raises.
"""

from __future__ import annotations

import ctypes
import math
import os
from typing import Optional

import torch

__all__ = [
    "load_library", "reshape_and_cache", "reshape_and_cache_fp8", "copy_blocks", "decode",
    "decode_fp8", "decode_cascade", "decode_cascade_fp8", "decode_cascade_workspace_bytes",
    "prefill_chunk", "prefill_chunk_fp8", "mixed_step", "decode_workspace_bytes",
    "prefill_workspace_bytes", "stream_read", "trace_enable", "trace_read", "PagedAttentionError",
    "pool_shape", "LIB_PATH", "set_tunable", "get_tunable", "tunables", "TUNABLES",
    "decode_no_alloc",
]

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libpagedattn.so")

PA_OK = 0
STATUS_NAMES = {1: "PA_ERR_NULL_POINTER", 2: "PA_ERR_INVALID_ARG", 3: "PA_ERR_UNSUPPORTED",
                4: "PA_ERR_WORKSPACE", 5: "PA_ERR_HIP"}


class PagedAttentionError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{STATUS_NAMES.get(status, status)}: {message}")
        self.status = status


_lib = None
_P = ctypes.c_void_p
_I32 = ctypes.c_int32
_I64 = ctypes.c_int64
_SZ = ctypes.c_size_t

class _PrefillArgs(ctypes.Structure):
    """pa_prefill_args (include/pa.h), field for field."""
    _fields_ = [("out", _P), ("query", _P), ("key_cache", _P), ("value_cache", _P),
                ("num_blocks", _I64), ("block_tables", _P), ("query_start_loc", _P),
                ("seq_lens", _P), ("num_seqs", _I32), ("total_q", _I32), ("max_q_len", _I32),
                ("num_q_heads", _I32), ("num_kv_heads", _I32), ("head_dim", _I32),
                ("block_size", _I32), ("max_blocks_per_seq", _I32), ("max_seq_len", _I32),
                ("scale", ctypes.c_float), ("kv_fp8", _I32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("workspace", _P), ("workspace_bytes", _SZ)]


class _DecodeArgs(ctypes.Structure):
    """pa_decode_args (include/pa.h), field for field."""
    _fields_ = [("out", _P), ("query", _P), ("key_cache", _P), ("value_cache", _P),
                ("num_blocks", _I64), ("block_tables", _P), ("seq_lens", _P), ("num_seqs", _I32),
                ("num_q_heads", _I32), ("num_kv_heads", _I32), ("head_dim", _I32),
                ("block_size", _I32), ("max_blocks_per_seq", _I32), ("max_seq_len", _I32),
                ("scale", ctypes.c_float), ("kv_fp8", _I32), ("k_scale", ctypes.c_float),
                ("v_scale", ctypes.c_float), ("workspace", _P), ("workspace_bytes", _SZ)]


_SIGNATURES = {
    "pa_version": (_I32, []),
    "pa_last_error": (ctypes.c_char_p, []),
    "pa_reshape_and_cache": (_I32, [_P, _P, _I64, _P, _P, _P, _I32, _I32, _I32, _I32, _I64, _P]),
    "pa_reshape_and_cache_fp8": (_I32, [_P, _P, _I64, _P, _P, _P, _I32, _I32, _I32, _I32, _I64,
                                        ctypes.c_float, ctypes.c_float, _P]),
    "pa_decode_fp8": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                             ctypes.c_float, ctypes.c_float, ctypes.c_float, _P, _SZ, _P]),
    "pa_decode_cascade_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pa_decode_cascade": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                 _I32, _I32, _I32, _I32, _I32, ctypes.c_float, _P, _SZ, _P]),
    "pa_decode_cascade_fp8": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _P, _P, _I32, _I32, _I32, _I32,
                                     _I32, _I32, _I32, _I32, _I32, _I32, ctypes.c_float,
                                     ctypes.c_float, ctypes.c_float, _P, _SZ, _P]),
    "pa_copy_blocks": (_I32, [_P, _P, _I64, _P, _I32, _I32, _I32, _I32, _P]),
    "pa_decode_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32]),
    "pa_decode_no_alloc": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32,
                                  _I32, ctypes.c_float, _P]),
    "pa_decode": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _I32, _I32, _I32, _I32, _I32, _I32, _I32,
                         ctypes.c_float, _P, _SZ, _P]),
    "pa_prefill_workspace_bytes": (_SZ, [_I32, _I32, _I32, _I32, _I32, _I32, _I32]),
    "pa_prefill_chunk": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                _I32, _I32, _I32, _I32, ctypes.c_float, _P, _SZ, _P]),
    "pa_prefill_chunk_fp8": (_I32, [_P, _P, _P, _P, _I64, _P, _P, _P, _I32, _I32, _I32, _I32, _I32,
                                    _I32, _I32, _I32, _I32, ctypes.c_float, ctypes.c_float,
                                    ctypes.c_float, _P, _SZ, _P]),
    "pa_stream_read_sink_words": (_I32, []),
    "pa_stream_read": (_I32, [_P, _SZ, _P, _SZ, _P]),
    "pa_mixed_step": (_I32, [ctypes.POINTER(_PrefillArgs), ctypes.POINTER(_DecodeArgs), _P, _P]),
    "pa_trace_enable": (_I32, [_I32]),
    "pa_set_tunable": (_I32, [ctypes.c_char_p, _I32]),
    "pa_get_tunable": (_I32, [ctypes.c_char_p, ctypes.POINTER(_I32)]),
    "pa_trace_read": (_I32, [ctypes.c_char_p, ctypes.POINTER(_I32), ctypes.POINTER(ctypes.c_double)]),
}


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the shared library (once).  Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m paged_kv_cache_444_amd.build_lib`")
    lib = ctypes.CDLL(path)
    for name, (res, args) in _SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib


def _check(status: int) -> None:
    if status != PA_OK:
        raise PagedAttentionError(status, load_library().pa_last_error().decode())


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _bf16(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must hold bf16 values (bfloat16 or a 16-bit integer view)")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    return t.data_ptr()


def _ints(t: torch.Tensor, dtype: torch.dtype, name: str) -> int:
    if not t.is_cuda or t.dtype != dtype or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU {dtype} tensor")
    return t.data_ptr()


def pool_shape(num_blocks: int, num_kv_heads: int, block_size: int, head_dim: int):
    """Shape of one K or V pool tensor: [num_blocks][num_kv_heads * block_size * head_dim]."""
    return (num_blocks, num_kv_heads * block_size * head_dim)


def _num_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor, num_kv_heads: int,
                block_size: int, head_dim: int) -> int:
    """Whole blocks both pools hold for this shape (the smaller of the two, so neither is read or
    written past its end).  Element counts are the same for bf16 and FP8 pools."""
    per = num_kv_heads * block_size * head_dim
    if per <= 0:
        raise ValueError("num_kv_heads, block_size and head_dim must be positive")
    n = min(key_cache.numel(), value_cache.numel()) // per
    if n < 1:
        raise ValueError(f"the pools must hold at least one block of {per} elements "
                         f"(key_cache {key_cache.numel()}, value_cache {value_cache.numel()})")
    return n


def _rows(t: torch.Tensor, n: int, name: str, *, dim0: Optional[int] = None) -> None:
    """Raise ValueError unless `t` has n elements (dim0 None) or n rows (dim0 = expected ndim)."""
    if dim0 is None:
        if t.numel() != n:
            raise ValueError(f"{name} must hold {n} entries (got {t.numel()})")
    elif t.dim() != dim0 or t.shape[0] != n:
        raise ValueError(f"{name} must be {dim0}-D with {n} rows (got shape {tuple(t.shape)})")


def _out_like(out: Optional[torch.Tensor], query: torch.Tensor) -> torch.Tensor:
    if out is None:
        return torch.empty_like(query)
    if out.shape != query.shape or out.element_size() != 2:
        raise ValueError(f"out must be a 16-bit tensor of the query's shape {tuple(query.shape)} "
                         f"(got {tuple(out.shape)}, {out.dtype})")
    return out


def _decode_shapes(query, block_tables, seq_lens) -> None:
    if query.dim() != 3:
        raise ValueError("query must be [num_seqs][num_q_heads][head_dim]")
    B = query.shape[0]
    _rows(seq_lens, B, "seq_lens")
    _rows(block_tables, B, "block_tables", dim0=2)


def _prefill_shapes(query, block_tables, query_start_loc, seq_lens) -> int:
    if query.dim() != 3:
        raise ValueError("query must be [total_q][num_q_heads][head_dim]")
    n = seq_lens.numel()
    _rows(query_start_loc, n + 1, "query_start_loc")
    _rows(block_tables, n, "block_tables", dim0=2)
    return n


def reshape_and_cache(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                      value_cache: torch.Tensor, slot_mapping: torch.Tensor, *, num_kv_heads: int,
                      head_dim: int, block_size: int) -> None:
    """Write key/value rows [T][Hkv][D] into the pools at `slot_mapping` (int64 [T], -1 = skip)."""
    lib = load_library()
    T = slot_mapping.numel()
    if key.shape != value.shape or key.numel() != T * num_kv_heads * head_dim:
        raise ValueError("key/value must be [T][num_kv_heads][head_dim]")
    n = _num_blocks(key_cache, value_cache, num_kv_heads, block_size, head_dim)
    _check(lib.pa_reshape_and_cache(_bf16(key, "key"), _bf16(value, "value"), num_kv_heads * head_dim,
                                    _bf16(key_cache, "key_cache"), _bf16(value_cache, "value_cache"),
                                    _ints(slot_mapping, torch.int64, "slot_mapping"), T, num_kv_heads,
                                    head_dim, block_size, n, _stream()))


def _fp8_pool(t: torch.Tensor, name: str) -> int:
    if not t.is_cuda or t.dtype != torch.uint8 or not t.is_contiguous():
        raise ValueError(f"{name} must be a contiguous GPU uint8 tensor of E4M3 codes")
    return t.data_ptr()


def reshape_and_cache_fp8(key: torch.Tensor, value: torch.Tensor, key_cache: torch.Tensor,
                          value_cache: torch.Tensor, slot_mapping: torch.Tensor, *, num_kv_heads: int,
                          head_dim: int, block_size: int, k_scale: float, v_scale: float) -> None:
    """reshape_and_cache into uint8 pools of E4M3 codes: code = E4M3(x / scale)."""
    lib = load_library()
    T = slot_mapping.numel()
    if key.shape != value.shape or key.numel() != T * num_kv_heads * head_dim:
        raise ValueError("key/value must be [T][num_kv_heads][head_dim]")
    n = _num_blocks(key_cache, value_cache, num_kv_heads, block_size, head_dim)
    _check(lib.pa_reshape_and_cache_fp8(_bf16(key, "key"), _bf16(value, "value"),
                                        num_kv_heads * head_dim, _fp8_pool(key_cache, "key_cache"),
                                        _fp8_pool(value_cache, "value_cache"),
                                        _ints(slot_mapping, torch.int64, "slot_mapping"), T,
                                        num_kv_heads, head_dim, block_size, n, float(k_scale),
                                        float(v_scale), _stream()))


def copy_blocks(key_cache: torch.Tensor, value_cache: torch.Tensor, block_mapping: torch.Tensor, *,
                num_kv_heads: int, head_dim: int, block_size: int) -> None:
    """Copy whole blocks of both pools: block_mapping int64 [n][2] of (source, destination) ids."""
    lib = load_library()
    if block_mapping.dim() != 2 or block_mapping.shape[1] != 2:
        raise ValueError("block_mapping must be [n][2]")
    n = _num_blocks(key_cache, value_cache, num_kv_heads, block_size, head_dim)
    _check(lib.pa_copy_blocks(_bf16(key_cache, "key_cache"), _bf16(value_cache, "value_cache"), n,
                              _ints(block_mapping, torch.int64, "block_mapping"),
                              block_mapping.shape[0], num_kv_heads, head_dim, block_size, _stream()))


def decode_workspace_bytes(num_seqs: int, num_q_heads: int, num_kv_heads: int, head_dim: int,
                           max_seq_len: int) -> int:
    """Workspace bytes pa_decode needs on the current device (0 for unsupported shapes)."""
    return int(load_library().pa_decode_workspace_bytes(num_seqs, num_q_heads, num_kv_heads, head_dim,
                                                        max_seq_len))


def prefill_workspace_bytes(num_seqs: int, total_q: int, max_q_len: int, num_q_heads: int,
                            num_kv_heads: int, head_dim: int, max_seq_len: int) -> int:
    """Workspace bytes pa_prefill_chunk needs on the current device (0: none)."""
    return int(load_library().pa_prefill_workspace_bytes(num_seqs, total_q, max_q_len, num_q_heads,
                                                         num_kv_heads, head_dim, max_seq_len))


def _workspace(nbytes: int, workspace: Optional[torch.Tensor], device) -> tuple:
    """Pointer and size of the workspace; a fresh one is zero-filled, as the library requires
    before a workspace's first use (a caller-provided one must have been zeroed once)."""
    if nbytes == 0:
        return 0, 0
    if workspace is None:
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    # A too-small workspace is passed through: the library reports PA_ERR_WORKSPACE.
    return workspace.data_ptr(), workspace.numel() * workspace.element_size()


def decode(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
           block_tables: torch.Tensor, seq_lens: torch.Tensor, *, num_kv_heads: int, block_size: int,
           scale: Optional[float] = None, max_seq_len: Optional[int] = None,
           out: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged decode attention: query [B][Hq][D] bf16 -> out [B][Hq][D] bf16.

    `max_seq_len` must bound seq_lens; if omitted it is read back from the device (a sync).
    """
    lib = load_library()
    _decode_shapes(query, block_tables, seq_lens)
    B, Hq, D = query.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    out = _out_like(out, query)
    n = _num_blocks(key_cache, value_cache, num_kv_heads, block_size, D)
    ws, ws_bytes = _workspace(decode_workspace_bytes(B, Hq, num_kv_heads, D, max_seq_len), workspace,
                              query.device)
    _check(lib.pa_decode(_bf16(out, "out"), _bf16(query, "query"), _bf16(key_cache, "key_cache"),
                         _bf16(value_cache, "value_cache"), n,
                         _ints(block_tables, torch.int32, "block_tables"),
                         _ints(seq_lens, torch.int32, "seq_lens"), B, Hq, num_kv_heads, D, block_size,
                         block_tables.shape[1], max_seq_len, float(scale), ws, ws_bytes, _stream()))
    return out


def decode_no_alloc(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                    block_tables: torch.Tensor, seq_lens: torch.Tensor, *, num_kv_heads: int,
                    block_size: int, max_seq_len: int, scale: Optional[float] = None,
                    out: Optional[torch.Tensor] = None) -> torch.Tensor:
    """`decode` without a workspace (pa_decode_no_alloc): the library's fixed per-device scratch
    array is used, so the call allocates nothing when `out` is given.  Calls that overlap in time
    on one device race on that array; batches too large for it raise PA_ERR_WORKSPACE."""
    lib = load_library()
    _decode_shapes(query, block_tables, seq_lens)
    B, Hq, D = query.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _out_like(out, query)
    n = _num_blocks(key_cache, value_cache, num_kv_heads, block_size, D)
    _check(lib.pa_decode_no_alloc(_bf16(out, "out"), _bf16(query, "query"),
                                  _bf16(key_cache, "key_cache"), _bf16(value_cache, "value_cache"),
                                  n, _ints(block_tables, torch.int32, "block_tables"),
                                  _ints(seq_lens, torch.int32, "seq_lens"), B, Hq, num_kv_heads, D,
                                  block_size, block_tables.shape[1], max_seq_len, float(scale),
                                  _stream()))
    return out


def decode_fp8(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
               block_tables: torch.Tensor, seq_lens: torch.Tensor, *, num_kv_heads: int,
               block_size: int, k_scale: float, v_scale: float, scale: Optional[float] = None,
               max_seq_len: Optional[int] = None, out: Optional[torch.Tensor] = None,
               workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Paged decode over uint8 pools of E4M3 codes (written by reshape_and_cache_fp8)."""
    lib = load_library()
    _decode_shapes(query, block_tables, seq_lens)
    B, Hq, D = query.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    out = _out_like(out, query)
    n = _num_blocks(key_cache, value_cache, num_kv_heads, block_size, D)
    ws, ws_bytes = _workspace(decode_workspace_bytes(B, Hq, num_kv_heads, D, max_seq_len), workspace,
                              query.device)
    _check(lib.pa_decode_fp8(_bf16(out, "out"), _bf16(query, "query"),
                             _fp8_pool(key_cache, "key_cache"), _fp8_pool(value_cache, "value_cache"),
                             n, _ints(block_tables, torch.int32, "block_tables"),
                             _ints(seq_lens, torch.int32, "seq_lens"), B, Hq, num_kv_heads, D,
                             block_size, block_tables.shape[1], max_seq_len, float(scale),
                             float(k_scale), float(v_scale), ws, ws_bytes, _stream()))
    return out


def decode_cascade_workspace_bytes(num_seqs: int, num_groups: int, max_group_size: int,
                                   num_q_heads: int, num_kv_heads: int, head_dim: int,
                                   max_prefix_len: int) -> int:
    """Workspace bytes pa_decode_cascade needs on the current device (0 for unsupported shapes)."""
    return int(load_library().pa_decode_cascade_workspace_bytes(
        num_seqs, num_groups, max_group_size, num_q_heads, num_kv_heads, head_dim, max_prefix_len))


def _cascade(fp8: bool, query, key_cache, value_cache, block_tables, seq_lens, group_start,
             prefix_lens, *, max_prefix_len, max_group_size, num_kv_heads, block_size, scale,
             max_seq_len, out, workspace, k_scale=1.0, v_scale=1.0):
    lib = load_library()
    _decode_shapes(query, block_tables, seq_lens)
    B, Hq, D = query.shape
    n_groups = group_start.numel() - 1
    if n_groups < 1 and B > 0:
        raise ValueError("group_start must hold num_groups + 1 >= 2 entries")
    _rows(prefix_lens, B, "prefix_lens")
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    if max_seq_len is None:
        max_seq_len = int(seq_lens.max().item()) if B else 0
    out = _out_like(out, query)
    nbytes = decode_cascade_workspace_bytes(B, n_groups, max_group_size, Hq, num_kv_heads, D,
                                            max_prefix_len)
    ws, ws_bytes = _workspace(nbytes, workspace, query.device)
    pools = ((_fp8_pool(key_cache, "key_cache"), _fp8_pool(value_cache, "value_cache")) if fp8 else
             (_bf16(key_cache, "key_cache"), _bf16(value_cache, "value_cache")))
    n = _num_blocks(key_cache, value_cache, num_kv_heads, block_size, D)
    args = [_bf16(out, "out"), _bf16(query, "query"), *pools, n,
            _ints(block_tables, torch.int32, "block_tables"), _ints(seq_lens, torch.int32, "seq_lens"),
            _ints(group_start, torch.int32, "group_start"),
            _ints(prefix_lens, torch.int32, "prefix_lens"), B, n_groups, max_group_size,
            max_prefix_len, Hq, num_kv_heads, D, block_size, block_tables.shape[1], max_seq_len,
            float(scale)]
    if fp8:
        _check(lib.pa_decode_cascade_fp8(*args, float(k_scale), float(v_scale), ws, ws_bytes,
                                         _stream()))
    else:
        _check(lib.pa_decode_cascade(*args, ws, ws_bytes, _stream()))
    return out


def decode_cascade(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                   block_tables: torch.Tensor, seq_lens: torch.Tensor, group_start: torch.Tensor,
                   prefix_lens: torch.Tensor, *, max_prefix_len: int, max_group_size: int,
                   num_kv_heads: int, block_size: int, scale: Optional[float] = None,
                   max_seq_len: Optional[int] = None, out: Optional[torch.Tensor] = None,
                   workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Decode of groups of sequences sharing the blocks of their first prefix_lens[s] tokens
    (group i is sequences group_start[i] .. group_start[i+1]-1): the same result as `decode`."""
    return _cascade(False, query, key_cache, value_cache, block_tables, seq_lens, group_start,
                    prefix_lens, max_prefix_len=max_prefix_len, max_group_size=max_group_size,
                    num_kv_heads=num_kv_heads, block_size=block_size, scale=scale,
                    max_seq_len=max_seq_len, out=out, workspace=workspace)


def decode_cascade_fp8(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                       block_tables: torch.Tensor, seq_lens: torch.Tensor,
                       group_start: torch.Tensor, prefix_lens: torch.Tensor, *,
                       max_prefix_len: int, max_group_size: int, num_kv_heads: int,
                       block_size: int, k_scale: float, v_scale: float,
                       scale: Optional[float] = None, max_seq_len: Optional[int] = None,
                       out: Optional[torch.Tensor] = None,
                       workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """decode_cascade over uint8 pools of E4M3 codes: the same result as `decode_fp8`."""
    return _cascade(True, query, key_cache, value_cache, block_tables, seq_lens, group_start,
                    prefix_lens, max_prefix_len=max_prefix_len, max_group_size=max_group_size,
                    num_kv_heads=num_kv_heads, block_size=block_size, scale=scale,
                    max_seq_len=max_seq_len, out=out, workspace=workspace, k_scale=k_scale,
                    v_scale=v_scale)


def prefill_chunk(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                  block_tables: torch.Tensor, query_start_loc: torch.Tensor, seq_lens: torch.Tensor, *,
                  num_kv_heads: int, block_size: int, max_q_len: int, max_seq_len: int,
                  scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                  workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Causal chunked-prefill attention: query [total_q][Hq][D] -> out [total_q][Hq][D] bf16."""
    lib = load_library()
    n = _prefill_shapes(query, block_tables, query_start_loc, seq_lens)
    total_q, Hq, D = query.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _out_like(out, query)
    nb = _num_blocks(key_cache, value_cache, num_kv_heads, block_size, D)
    ws, ws_bytes = _workspace(prefill_workspace_bytes(n, total_q, max_q_len, Hq, num_kv_heads, D,
                                                      max_seq_len), workspace, query.device)
    _check(lib.pa_prefill_chunk(_bf16(out, "out"), _bf16(query, "query"), _bf16(key_cache, "key_cache"),
                                _bf16(value_cache, "value_cache"), nb,
                                _ints(block_tables, torch.int32, "block_tables"),
                                _ints(query_start_loc, torch.int32, "query_start_loc"),
                                _ints(seq_lens, torch.int32, "seq_lens"), n, total_q, max_q_len, Hq,
                                num_kv_heads, D, block_size, block_tables.shape[1], max_seq_len,
                                float(scale), ws, ws_bytes, _stream()))
    return out


_side_streams = {}


def _owned_workspace(nbytes: int, workspace: Optional[torch.Tensor], device):
    """(tensor, pointer, bytes) of a workspace; a fresh one is zero-filled.  The caller keeps the
    tensor: two workspaces used by concurrent kernels must not share a cached block."""
    if nbytes == 0:
        return None, 0, 0
    if workspace is None:
        workspace = torch.zeros(nbytes, dtype=torch.uint8, device=device)
    return workspace, workspace.data_ptr(), workspace.numel() * workspace.element_size()


def _pools(key_cache, value_cache, fp8):
    if fp8:
        return _fp8_pool(key_cache, "key_cache"), _fp8_pool(value_cache, "value_cache")
    return _bf16(key_cache, "key_cache"), _bf16(value_cache, "value_cache")


def mixed_step(prefill: dict, decode_call: dict, *, side_stream=None, fp8: bool = False):
    """One chunked-prefill batch step (pa_mixed_step): the prefill chunk and the decode of the
    other sequences run side by side on two streams, so decode's HBM-bound work overlaps the
    matrix-core-bound chunk.

    `prefill` and `decode_call` hold the keyword arguments of `prefill_chunk` and `decode` (with
    `fp8`: of `prefill_chunk_fp8` and `decode_fp8`, the uint8 pools and k_scale / v_scale).  Both
    halves start after the work already queued on the current stream (write every new token's
    K/V with reshape_and_cache first), and the current stream waits for both.  The decode runs on
    `side_stream` (default: one stream per device, kept for reuse).  Returns (prefill output,
    decode output), bit for bit those of the two calls made one after the other.
    """
    lib = load_library()
    main = torch.cuda.current_stream()
    if side_stream is None:
        side_stream = _side_streams.get(main.device)
        if side_stream is None:
            side_stream = _side_streams[main.device] = torch.cuda.Stream(device=main.device)
    p, d = dict(prefill), dict(decode_call)
    # prefill half
    pq = p["query"]
    n_p = _prefill_shapes(pq, p["block_tables"], p["query_start_loc"], p["seq_lens"])
    total_q, Hq, D = pq.shape
    pout = _out_like(p.get("out"), pq)
    pws_t, pws, pws_bytes = _owned_workspace(
        prefill_workspace_bytes(n_p, total_q, p["max_q_len"], Hq, p["num_kv_heads"], D,
                                p["max_seq_len"]), p.get("workspace"), pq.device)
    nb = _num_blocks(p["key_cache"], p["value_cache"], p["num_kv_heads"], p["block_size"], D)
    pk, pv = _pools(p["key_cache"], p["value_cache"], fp8)
    pa_args = _PrefillArgs(
        _bf16(pout, "out"), _bf16(pq, "query"), pk, pv, nb,
        _ints(p["block_tables"], torch.int32, "block_tables"),
        _ints(p["query_start_loc"], torch.int32, "query_start_loc"),
        _ints(p["seq_lens"], torch.int32, "seq_lens"), n_p, total_q, p["max_q_len"], Hq,
        p["num_kv_heads"], D, p["block_size"], p["block_tables"].shape[1], p["max_seq_len"],
        float(p.get("scale") or 1.0 / math.sqrt(D)), int(fp8), float(p.get("k_scale", 1.0)),
        float(p.get("v_scale", 1.0)), pws, pws_bytes)
    # decode half
    dq = d["query"]
    _decode_shapes(dq, d["block_tables"], d["seq_lens"])
    B, dHq, dD = dq.shape
    max_len = d.get("max_seq_len")
    if max_len is None:
        max_len = int(d["seq_lens"].max().item()) if B else 0
    dout = _out_like(d.get("out"), dq)
    dws_t, dws, dws_bytes = _owned_workspace(
        decode_workspace_bytes(B, dHq, d["num_kv_heads"], dD, max_len), d.get("workspace"),
        dq.device)
    dnb = _num_blocks(d["key_cache"], d["value_cache"], d["num_kv_heads"], d["block_size"], dD)
    dk, dv = _pools(d["key_cache"], d["value_cache"], fp8)
    de_args = _DecodeArgs(
        _bf16(dout, "out"), _bf16(dq, "query"), dk, dv, dnb,
        _ints(d["block_tables"], torch.int32, "block_tables"),
        _ints(d["seq_lens"], torch.int32, "seq_lens"), B, dHq, d["num_kv_heads"], dD,
        d["block_size"], d["block_tables"].shape[1], max_len,
        float(d.get("scale") or 1.0 / math.sqrt(dD)), int(fp8), float(d.get("k_scale", 1.0)),
        float(d.get("v_scale", 1.0)), dws, dws_bytes)
    _check(lib.pa_mixed_step(ctypes.byref(pa_args), ctypes.byref(de_args), _stream(),
                             side_stream.cuda_stream))
    # Everything above was allocated on the current stream, which waits for the side stream
    # before any later work, so once the call is enqueued the workspaces may go back to the
    # cache: no later allocation can reach them before both halves are done.
    del pws_t, dws_t
    return pout, dout


def prefill_chunk_fp8(query: torch.Tensor, key_cache: torch.Tensor, value_cache: torch.Tensor,
                      block_tables: torch.Tensor, query_start_loc: torch.Tensor,
                      seq_lens: torch.Tensor, *, num_kv_heads: int, block_size: int, max_q_len: int,
                      max_seq_len: int, k_scale: float, v_scale: float,
                      scale: Optional[float] = None, out: Optional[torch.Tensor] = None,
                      workspace: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Chunked-prefill attention over uint8 pools of E4M3 codes (reshape_and_cache_fp8)."""
    lib = load_library()
    n = _prefill_shapes(query, block_tables, query_start_loc, seq_lens)
    total_q, Hq, D = query.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = _out_like(out, query)
    nb = _num_blocks(key_cache, value_cache, num_kv_heads, block_size, D)
    ws, ws_bytes = _workspace(prefill_workspace_bytes(n, total_q, max_q_len, Hq, num_kv_heads, D,
                                                      max_seq_len), workspace, query.device)
    _check(lib.pa_prefill_chunk_fp8(_bf16(out, "out"), _bf16(query, "query"),
                                    _fp8_pool(key_cache, "key_cache"),
                                    _fp8_pool(value_cache, "value_cache"), nb,
                                    _ints(block_tables, torch.int32, "block_tables"),
                                    _ints(query_start_loc, torch.int32, "query_start_loc"),
                                    _ints(seq_lens, torch.int32, "seq_lens"), n, total_q, max_q_len,
                                    Hq, num_kv_heads, D, block_size, block_tables.shape[1],
                                    max_seq_len, float(scale), float(k_scale), float(v_scale), ws,
                                    ws_bytes, _stream()))
    return out


def stream_read(buf: torch.Tensor, sink: Optional[torch.Tensor] = None) -> torch.Tensor:
    """Read every byte of `buf` once (the streaming-read ceiling kernel); returns the sink."""
    lib = load_library()
    if not buf.is_cuda or not buf.is_contiguous():
        raise ValueError("buf must be a contiguous GPU tensor")
    words = int(lib.pa_stream_read_sink_words())
    if sink is None:
        sink = torch.empty(max(words, 1), dtype=torch.int32, device=buf.device)
    _check(lib.pa_stream_read(buf.data_ptr(), buf.numel() * buf.element_size(), sink.data_ptr(),
                              sink.numel(), _stream()))
    return sink


def trace_enable(on: bool = True) -> None:
    _check(load_library().pa_trace_enable(1 if on else 0))


def trace_read(kernel_name: str):
    """(launches, total_ms) recorded for `kernel_name` since the last read; forgets them."""
    n = _I32()
    ms = ctypes.c_double()
    _check(load_library().pa_trace_read(kernel_name.encode(), ctypes.byref(n), ctypes.byref(ms)))
    return n.value, ms.value


# Launch tunables of the library (include/pa.h): they change how work is spread over the GPU,
# never what is computed beyond fp32 rounding order.
TUNABLES = ("PA_DECODE_PREFETCH", "PA_DECODE_PREFETCH_FP8", "PA_DECODE_MFMA", "PA_DECODE_QUAD",
            "PA_DECODE_PIECE_COST", "PA_DECODE_WORKERS", "PA_DECODE_STATIC_Q10", "PA_DECODE_CHUNK",
            "PA_PREFILL_SPLITS", "PA_DECODE_TAIL_Q10", "PA_DECODE_TAIL_Q10_FP8",
            "PA_DECODE_TAIL_CHUNK")


def set_tunable(name: str, value: int) -> None:
    """Set a launch tunable (PagedAttentionError for an unknown name or out-of-range value)."""
    _check(load_library().pa_set_tunable(name.encode(), int(value)))


def get_tunable(name: str) -> int:
    v = _I32()
    _check(load_library().pa_get_tunable(name.encode(), ctypes.byref(v)))
    return v.value


class tunables:
    """Context manager: set launch tunables for a block, then restore their previous values.

        with pa.tunables(PA_DECODE_WORKERS=8, PA_DECODE_MFMA=0):
            pa.decode(...)
    """

    def __init__(self, **values: int):
        self._values = values
        self._saved = {}

    def __enter__(self):
        for k, v in self._values.items():
            self._saved[k] = get_tunable(k)
            set_tunable(k, v)
        return self

    def __exit__(self, *exc):
        for k, v in self._saved.items():
            set_tunable(k, v)
        return False
