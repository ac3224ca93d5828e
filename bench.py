"""Benchmark: paged decode attention at the Llama-3.3-70B shape, batch 128, on one MI355X.

One step = one pa_decode call over 128 sequences (64 query / 8 KV heads, head_dim 128, 16-token
blocks, lognormal context lengths with mean 1,500 and standard deviation 600 clipped to
[16, 8192]) whose K/V, queries and tables are already resident in HBM.  Consecutive steps cycle
through `--layers` distinct copies of the KV pools, as consecutive decode calls of a model touch
different layers' caches, so a step cannot be served from the 256 MB last-level cache that the
previous step filled.  Prints one JSON line.

  value        algorithmic bytes of one call / wall time per step (GB/s)
  roofline     the dominant kernel (decode_kernel): algorithmic bytes per launch / its mean
               event-timed duration over the timed steps, against the 8 TB/s HBM peak
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same batch (a correctness tool,
               not an optimised CPU kernel)

`--mode copy` instead times a plain device-to-device copy of a known size: the calibration run for
the FETCH_SIZE / WRITE_SIZE hardware counters.
"""

from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
METRIC = "pa_decode achieved HBM GB/s (% of peak) + seqs/s, 70B-shape B=128"


def decode_bytes(seq_lens, Hq, Hkv, D, bs):
    """Algorithmic HBM bytes of one decode call: each sequence's K and V once, its query read and
    output written once, its used block-table entries and its length."""
    L = np.asarray(seq_lens, dtype=np.int64)
    kv = int((L * Hkv * D * 2 * 2).sum())
    qo = len(L) * 2 * Hq * D * 2
    tables = int(((L + bs - 1) // bs).sum()) * 4 + len(L) * 4
    return kv + qo + tables


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--layers", type=int, default=4,
                    help="distinct KV pool copies cycled through by consecutive steps")
    ap.add_argument("--warm-steps", type=int, default=50,
                    help="extra steps on one pool (cache-warm), reported for context")
    ap.add_argument("--cpu-seconds", type=float, default=10.0,
                    help="repeat the oracle over the whole batch until this much CPU time is spent")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--mode", choices=["decode", "copy"], default="decode")
    ap.add_argument("--copy-mib", type=int, default=1024)
    return ap.parse_args()


def log(msg):
    print(f"bench: {msg}", file=sys.stderr, flush=True)


def run_copy(args):
    """Plain copy of --copy-mib MiB, repeated: reads and writes exactly that many bytes per launch."""
    import torch

    n = args.copy_mib << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        dst.copy_(src)
    torch.cuda.synchronize()
    dt = (time.perf_counter() - t0) / args.steps
    print(json.dumps({"mode": "copy", "bytes_read_per_launch": n, "bytes_written_per_launch": n,
                      "launches": args.steps + 3, "us_per_copy": round(dt * 1e6, 2),
                      "gbs_read_plus_write": round(2 * n / dt / 1e9, 1)}), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              f"(this build runs on a single GPU: run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    if args.mode == "copy":
        run_copy(args)
        return

    import paged_kv_cache_444_amd as pa
    from workloads import named_case

    log("generating the 70B-shape batch-128 decode workload")
    case = named_case(2)
    d = case.decode
    Hq, Hkv, D, bs = case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    B = d.num_seqs
    max_len = d.max_seq_len

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    kc0, vc0 = dev(case.key_cache), dev(case.value_cache)
    pools = [(kc0, vc0)] + [(kc0.clone(), vc0.clone()) for _ in range(max(args.layers, 1) - 1)]
    q = dev(d.query)
    bt = torch.from_numpy(d.block_tables).cuda()
    sl = torch.from_numpy(d.seq_lens).cuda()
    out = torch.empty_like(q)
    ws = torch.zeros(max(pa.decode_workspace_bytes(B, Hq, Hkv, D, max_len), 1), dtype=torch.uint8,
                     device="cuda")
    scale = float(case.scale)

    def step(i):
        kc, vc = pools[i % len(pools)]
        pa.decode(q, kc, vc, bt, sl, num_kv_heads=Hkv, block_size=bs, scale=scale,
                  max_seq_len=max_len, out=out, workspace=ws)

    log(f"warmup {args.warmup} steps over {len(pools)} pool copies")
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    pa.trace_enable(True)
    for name in ("decode_partition", "decode_merge"):
        pa.trace_read(name)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    n_main, ms_main = pa.trace_read("decode_partition")
    n_merge, ms_merge = pa.trace_read("decode_merge")
    log(f"timed {args.steps} steps")

    warm_us = None
    if args.warm_steps > 0:
        for _ in range(5):
            step(0)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        for _ in range(args.warm_steps):
            step(0)
        torch.cuda.synchronize()
        warm_us = (time.perf_counter() - w0) * 1e6 / args.warm_steps
        pa.trace_read("decode_partition")
        pa.trace_read("decode_merge")
    pa.trace_enable(False)

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    nbytes = decode_bytes(d.seq_lens, Hq, Hkv, D, bs)
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    main_ms = ms_main / max(n_main, 1)
    main_gbs = nbytes / (main_ms * 1e-3) / 1e9

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on a sample")
        cpu = cpu_baseline(case, args.cpu_seconds)

    rec = {
        "metric": METRIC,
        "value": round(gbs, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(B / (ms_per_step * 1e-3), 1),
        "config": {
            "workload": case.name, "num_seqs": B, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "head_dim": D, "block_size": bs, "mean_seq_len": round(float(d.seq_lens.mean()), 1),
            "max_seq_len": max_len, "algorithmic_bytes": nbytes, "pool_blocks": case.num_blocks,
            "pool_copies_cycled": len(pools),
            "decode_workers": int(os.environ.get("PA_DECODE_WORKERS", "0")) or "default",
            "decode_prefetch": int(os.environ.get("PA_DECODE_PREFETCH", "1")),
            "decode_static_q10": int(os.environ.get("PA_DECODE_STATIC_Q10", "1024")),
            "decode_chunk_steps": int(os.environ.get("PA_DECODE_CHUNK", "4")),
        },
        "roofline": {
            "bound": "hbm", "kernel": "decode_kernel", "achieved": round(main_gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(main_gbs / HBM_PEAK_GBS, 4),
            "traffic": None, "launch_us": round(main_ms * 1e3, 2),
            "merge_launch_us": round(ms_merge / max(n_merge, 1) * 1e3, 2),
        },
        "warm_single_pool_us_per_step": None if warm_us is None else round(warm_us, 2),
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(case, budget_s):
    """Time the fp64 oracle over the whole batch (all sequences and heads), repeated until about
    `budget_s` seconds have passed (at most 8 runs); report the median run.  np.einsum without
    optimize runs single-threaded, so one core does the work."""
    from oracle import paged_attention as oracle

    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    d = case.decode
    runs = []
    while len(runs) < 8 and sum(runs) < budget_s:
        t0 = time.perf_counter()
        oracle.decode(d.query, case.key_cache, case.value_cache, d.block_tables, d.seq_lens,
                      case.num_kv_heads, case.head_dim, case.block_size, case.scale)
        runs.append(time.perf_counter() - t0)
    dt = float(np.median(runs))
    nbytes = decode_bytes(d.seq_lens, case.num_q_heads, case.num_kv_heads, case.head_dim,
                          case.block_size)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "host_cores_available": cores, "seconds_per_call": round(dt, 3), "runs": len(runs),
            "seqs_per_s": round(d.num_seqs / dt, 2),
            "sample": f"the whole batch ({d.num_seqs} sequences, {case.num_q_heads} query heads), "
                      f"median of {len(runs)} runs; fp64 NumPy gather + einsum, single-threaded"}


if __name__ == "__main__":
    main()
