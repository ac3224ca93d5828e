"""The C ABI on the CPU: the library loads, exports every entry point include/pa.h declares, and
rejects bad host-side arguments before touching the GPU (no kernel is launched here)."""

import ctypes
import os
import re

import pytest

import paged_kv_cache_444_amd as pa

HEADER = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "include", "pa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(pa_[a-z0-9_]+)\s*\(", text)))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(pa.LIB_PATH):
        pytest.fail("libpagedattn.so is not built (run __graft_entry__.build())")
    return pa.load_library()


def test_every_declared_symbol_is_exported(lib):
    names = declared_functions()
    assert {"pa_reshape_and_cache", "pa_decode", "pa_prefill_chunk"} <= set(names)
    for n in names:
        assert hasattr(lib, n), n


def test_version_and_error_text(lib):
    assert lib.pa_version() >= 200
    assert isinstance(lib.pa_last_error(), bytes)


def test_workspace_queries_reject_unsupported_shapes(lib):
    # Sizes of supported shapes depend on the device (GPU tests check them); unsupported or empty
    # shapes report 0 without touching a device.
    assert lib.pa_decode_workspace_bytes(0, 64, 8, 128, 8192) == 0
    assert lib.pa_decode_workspace_bytes(128, 64, 6, 128, 8192) == 0   # Hq % Hkv
    assert lib.pa_decode_workspace_bytes(128, 64, 8, 96, 8192) == 0    # head_dim
    assert lib.pa_decode_workspace_bytes(128, 64, 2, 128, 8192) == 0   # group 32


def test_host_side_validation(lib):
    # Each call fails validation before any device work: statuses follow include/pa.h.
    z = 0
    assert lib.pa_decode(z, z, z, z, 1000, z, z, 1, 6, 4, 128, 16, 4, 64, 0.1, z, 0, z) == 2   # Hq % Hkv
    assert lib.pa_decode(z, z, z, z, 1000, z, z, 1, 8, 2, 96, 16, 4, 64, 0.1, z, 0, z) == 3    # head_dim
    assert lib.pa_decode(z, z, z, z, 1000, z, z, 1, 8, 2, 128, 8, 4, 64, 0.1, z, 0, z) == 3    # block size
    assert lib.pa_decode(z, z, z, z, 1000, z, z, 1, 64, 2, 128, 16, 4, 64, 0.1, z, 0, z) == 3  # group 32
    assert lib.pa_decode(z, z, z, z, 1000, z, z, 1, 8, 2, 128, 16, 4, 65, 0.1, z, 0, z) == 2   # L > table
    assert lib.pa_decode(z, z, z, z, 1000, z, z, 1, 8, 2, 128, 16, 4, 64, float("inf"), z, 0, z) == 2
    assert lib.pa_decode(z, z, z, z, 1000, z, z, 1, 8, 2, 128, 16, 4, 64, 0.1, z, 0, z) == 1   # nulls
    assert lib.pa_decode(z, z, z, z, 1000, z, z, -1, 8, 2, 128, 16, 4, 64, 0.1, z, 0, z) == 2
    assert lib.pa_decode(z, z, z, z, 1000, z, z, 0, 8, 2, 128, 16, 4, 64, 0.1, z, 0, z) == 0   # empty
    assert lib.pa_decode(z, z, z, z, 1000, z, z, 1, 6, 4, 128, 16, 4, 64, 0.1, z, 0, z) == 2
    assert b"not a multiple" in lib.pa_last_error()
    assert lib.pa_reshape_and_cache(z, z, 256, z, z, z, 1, 2, 128, 16, 10, z) == 1
    assert lib.pa_reshape_and_cache(z, z, 100, z, z, z, 1, 2, 128, 16, 10, z) == 2     # stride
    assert lib.pa_reshape_and_cache(z, z, 256, z, z, z, 0, 2, 128, 16, 10, z) == 0     # no tokens
    assert lib.pa_reshape_and_cache(z, z, 256, z, z, z, 1, 2, 128, 16, 0, z) == 2      # no blocks
    assert lib.pa_copy_blocks(z, z, 10, z, 1, 2, 128, 16, z) == 1                  # nulls
    assert lib.pa_copy_blocks(z, z, 10, z, -1, 2, 128, 16, z) == 2                 # pairs
    assert lib.pa_copy_blocks(z, z, 10, z, 1, 2, 96, 16, z) == 3                   # head_dim
    assert lib.pa_copy_blocks(z, z, 0, z, 1, 2, 128, 16, z) == 2                   # no blocks
    assert lib.pa_copy_blocks(z, z, 10, z, 0, 2, 128, 16, z) == 0                  # no pairs
    # FP8 entry points: scales must be finite and positive
    assert lib.pa_decode_fp8(z, z, z, z, 10, z, z, 1, 8, 2, 128, 16, 4, 64, 0.1, 0.0, 1.0, z, 0, z) == 2
    assert lib.pa_decode_fp8(z, z, z, z, 10, z, z, 1, 8, 2, 128, 16, 4, 64, 0.1, 1.0, float("nan"),
                             z, 0, z) == 2
    assert lib.pa_decode_fp8(z, z, z, z, 10, z, z, 1, 8, 2, 96, 16, 4, 64, 0.1, 1.0, 1.0, z, 0, z) == 3
    assert lib.pa_reshape_and_cache_fp8(z, z, 256, z, z, z, 1, 2, 128, 16, 10, -1.0, 1.0, z) == 2
    assert lib.pa_reshape_and_cache_fp8(z, z, 256, z, z, z, 0, 2, 128, 16, 10, 1.0, 1.0, z) == 0
    # cascade: max_prefix_len beyond max_seq_len / negative; null pointers; FP8 scale
    assert lib.pa_decode_cascade(z, z, z, z, 10, z, z, z, z, 4, 1, 4, 80, 8, 2, 64, 16, 8, 64, 0.1,
                                 z, 0, z) == 2
    assert lib.pa_decode_cascade(z, z, z, z, 10, z, z, z, z, 4, 1, 4, -16, 8, 2, 64, 16, 4, 64, 0.1,
                                 z, 0, z) == 2
    assert lib.pa_decode_cascade(z, z, z, z, 10, z, z, z, z, 4, 1, 4, 32, 8, 2, 64, 16, 4, 64, 0.1,
                                 z, 0, z) == 1
    assert lib.pa_decode_cascade_fp8(z, z, z, z, 10, z, z, z, z, 4, 1, 4, 32, 8, 2, 64, 16, 4, 64,
                                     0.1, 0.0, 1.0, z, 0, z) == 2
    assert lib.pa_decode_cascade_workspace_bytes(4, 1, 4, 8, 2, 96, 32) == 0
    assert lib.pa_prefill_chunk_fp8(z, z, z, z, 10, z, z, z, 1, 4, 4, 8, 2, 64, 16, 4, 64, 0.1, 0.0,
                                    1.0, z, 0, z) == 2  # k_scale
    # the no-allocation decode: pa_decode's host checks, no workspace
    assert lib.pa_decode_no_alloc(z, z, z, z, 1000, z, z, 1, 6, 4, 128, 16, 4, 64, 0.1, z) == 2
    assert lib.pa_decode_no_alloc(z, z, z, z, 1000, z, z, 1, 8, 2, 96, 16, 4, 64, 0.1, z) == 3
    assert lib.pa_decode_no_alloc(z, z, z, z, 1000, z, z, 1, 8, 2, 128, 16, 4, 64, 0.1, z) == 1
    assert lib.pa_decode_no_alloc(z, z, z, z, 1000, z, z, 0, 8, 2, 128, 16, 4, 64, 0.1, z) == 0
    assert lib.pa_stream_read(z, 0, z, 0, z) == 0       # nothing to read
    assert lib.pa_stream_read(z, 32, z, 0, z) == 1      # nulls
    assert lib.pa_trace_read(b"decode_partition", None, None) == 1


def test_argument_structs_match_the_header(tmp_path):
    """pa_prefill_args / pa_decode_args: the binding's ctypes mirrors have the header's field
    offsets and sizes (the header compiled by the host C compiler)."""
    import shutil
    import subprocess

    cc = shutil.which("gcc") or shutil.which("cc")
    if cc is None:
        pytest.skip("no host C compiler")
    lines = ["#include <stdio.h>", "#include <stddef.h>", '#include "pa.h"', "int main(void) {"]
    for cname, cls in (("pa_prefill_args", pa._PrefillArgs), ("pa_decode_args", pa._DecodeArgs)):
        lines.append(f'  printf("{cname} size %zu\\n", sizeof({cname}));')
        for f, _ in cls._fields_:
            lines.append(f'  printf("{cname} {f} %zu\\n", offsetof({cname}, {f}));')
    lines += ["  return 0;", "}"]
    src = tmp_path / "abi.c"
    src.write_text("\n".join(lines))
    exe = tmp_path / "abi"
    subprocess.run([cc, "-I", os.path.dirname(HEADER), str(src), "-o", str(exe)], check=True)
    out = subprocess.run([str(exe)], check=True, capture_output=True, text=True).stdout.split("\n")
    want = {}
    for cname, cls in (("pa_prefill_args", pa._PrefillArgs), ("pa_decode_args", pa._DecodeArgs)):
        want[f"{cname} size"] = ctypes.sizeof(cls)
        for f, _ in cls._fields_:
            want[f"{cname} {f}"] = getattr(cls, f).offset
    got = {l.rsplit(" ", 1)[0]: int(l.rsplit(" ", 1)[1]) for l in out if l}
    assert got == want


def test_binding_exports_every_listed_name():
    assert [n for n in pa.__all__ if not hasattr(pa, n)] == []


def test_mixed_step_with_empty_halves(lib):
    """Empty halves (no sequences) may pass null pointers: with both empty the call succeeds on
    one stream without launching anything; a bad shape in either half is still rejected."""
    def prefill_args(num_seqs=0, head_dim=128, out=None):
        return pa._PrefillArgs(out=out, num_blocks=16, num_seqs=num_seqs, total_q=num_seqs,
                               max_q_len=num_seqs, num_q_heads=8, num_kv_heads=2,
                               head_dim=head_dim, block_size=16, max_blocks_per_seq=4,
                               max_seq_len=64, scale=0.125, k_scale=1.0, v_scale=1.0)

    def decode_args(num_seqs=0, head_dim=128, out=None):
        return pa._DecodeArgs(out=out, num_blocks=16, num_seqs=num_seqs, num_q_heads=8,
                              num_kv_heads=2, head_dim=head_dim, block_size=16,
                              max_blocks_per_seq=4, max_seq_len=64, scale=0.125, k_scale=1.0,
                              v_scale=1.0)

    def call(pf, dc):
        return lib.pa_mixed_step(ctypes.byref(pf), ctypes.byref(dc), None, None)

    assert call(prefill_args(), decode_args()) == 0, lib.pa_last_error()
    assert call(prefill_args(head_dim=96), decode_args()) == 3  # unsupported head_dim
    assert call(prefill_args(), decode_args(head_dim=96)) == 3
    assert call(prefill_args(num_seqs=-1), decode_args()) == 2


def test_mixed_step_rejects_overlapping_outputs_and_workspaces(lib):
    """The two halves of a mixed step run at the same time, so no byte one writes may be written
    by the other: outputs and used workspace ranges must be disjoint (checked on the host before
    any launch; the pointers here are never dereferenced)."""
    Hq, Hkv, D = 64, 8, 128
    L, q = 40000, 512  # longer than one workgroup's table slice: always split, on any device

    def prefill_args(out, ws, ws_bytes):
        return pa._PrefillArgs(out=out, query=0x100000, key_cache=0x200000, value_cache=0x300000,
                               num_blocks=4096, block_tables=0x400000, query_start_loc=0x410000,
                               seq_lens=0x420000, num_seqs=1, total_q=q, max_q_len=q,
                               num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D, block_size=16,
                               max_blocks_per_seq=L // 16, max_seq_len=L, scale=0.088,
                               k_scale=1.0, v_scale=1.0, workspace=ws, workspace_bytes=ws_bytes)

    def decode_args(out):
        return pa._DecodeArgs(out=out, query=0x500000, key_cache=0x200000, value_cache=0x300000,
                              num_blocks=4096, block_tables=0x600000, seq_lens=0x610000,
                              num_seqs=4, num_q_heads=Hq, num_kv_heads=Hkv, head_dim=D,
                              block_size=16, max_blocks_per_seq=64, max_seq_len=1024, scale=0.088,
                              k_scale=1.0, v_scale=1.0)

    need = lib.pa_prefill_workspace_bytes(1, q, q, Hq, Hkv, D, L)
    assert need > 0  # the long context is split, so the prefill half uses its workspace
    pout, ws = 0x10000000, 0x20000000
    out_bytes = q * Hq * D * 2

    def call(pf, dc):
        return lib.pa_mixed_step(ctypes.byref(pf), ctypes.byref(dc), None, None)

    # the decode output starts inside the prefill output
    assert call(prefill_args(pout, ws, need), decode_args(pout + out_bytes - 256)) == 2
    assert b"prefill output overlaps the decode output" in lib.pa_last_error()
    # the decode output lies inside the prefill workspace
    assert call(prefill_args(pout, ws, need), decode_args(ws + need // 2)) == 2
    assert b"prefill workspace overlaps the decode output" in lib.pa_last_error()
    # the prefill workspace runs into its own output
    assert call(prefill_args(ws + 256, ws, need), decode_args(0x30000000)) == 2


def test_tunable_setter(lib):
    """Launch tunables: read through pa_get_tunable, changed by pa_set_tunable within their range,
    rejected (and left unchanged) outside it or under an unknown name."""
    v = ctypes.c_int32()
    assert lib.pa_get_tunable(b"PA_DECODE_PIECE_COST", ctypes.byref(v)) == 0
    before = v.value
    assert lib.pa_set_tunable(b"PA_DECODE_PIECE_COST", 9) == 0
    assert lib.pa_get_tunable(b"PA_DECODE_PIECE_COST", ctypes.byref(v)) == 0 and v.value == 9
    assert lib.pa_set_tunable(b"PA_DECODE_PIECE_COST", 65) == 2      # out of range
    assert b"PA_DECODE_PIECE_COST" in lib.pa_last_error()
    assert lib.pa_get_tunable(b"PA_DECODE_PIECE_COST", ctypes.byref(v)) == 0 and v.value == 9
    assert lib.pa_set_tunable(b"PA_NO_SUCH_THING", 1) == 2
    assert lib.pa_get_tunable(b"PA_NO_SUCH_THING", ctypes.byref(v)) == 2
    assert lib.pa_set_tunable(None, 1) == 1
    assert lib.pa_set_tunable(b"PA_DECODE_PIECE_COST", before) == 0
    # every name the binding lists is known to the library, and the context manager restores
    for name in pa.TUNABLES:
        assert lib.pa_get_tunable(name.encode(), ctypes.byref(v)) == 0, name
    with pa.tunables(PA_PREFILL_SPLITS=3, PA_DECODE_MFMA=0):
        assert pa.get_tunable("PA_PREFILL_SPLITS") == 3 and pa.get_tunable("PA_DECODE_MFMA") == 0
    assert pa.get_tunable("PA_PREFILL_SPLITS") == 0 and pa.get_tunable("PA_DECODE_MFMA") == 1


def test_tunables_read_from_the_environment_once():
    """A fresh process picks its tunables from the environment when the library first needs
    them; later changes of the environment do not matter."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    code = ("import os, paged_kv_cache_444_amd as pa\n"
            "a = pa.get_tunable('PA_DECODE_CHUNK'), pa.get_tunable('PA_DECODE_QUAD')\n"
            "os.environ['PA_DECODE_CHUNK'] = '7'\n"
            "print(a, pa.get_tunable('PA_DECODE_CHUNK'))\n")
    env = dict(os.environ, PA_DECODE_CHUNK="16", PA_DECODE_QUAD="9")  # 9: out of range, ignored
    r = subprocess.run([sys.executable, "-c", code], cwd=root, env=env, capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "(16, 1) 16"


def test_bench_refuses_more_than_one_gpu():
    """bench.py measures one GPU: --gpus above 1 exits with status 2 and says so, before any GPU
    or library work."""
    import subprocess
    import sys

    root = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
    r = subprocess.run([sys.executable, os.path.join(root, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr and r.stdout == ""
