"""Benchmark: paged decode attention at the Llama-3.3-70B shape, batch 128, on one MI355X.

One step = one pa_decode call over 128 sequences (64 query / 8 KV heads, head_dim 128, 16-token
blocks, lognormal context lengths with mean 1,500 clipped to [16, 8192]) whose K/V, queries and
tables are already resident in HBM.  Prints one JSON line.

  value        algorithmic bytes of the call / wall time per step, in GB/s
  roofline     the dominant kernel (decode_partition): algorithmic bytes per launch / its mean
               event-timed duration, against the 8 TB/s HBM peak
  cpu_baseline the fp64 CPU oracle on a bounded sample of the same batch (a correctness tool,
               not an optimised CPU kernel)
"""

from __future__ import annotations

import argparse
import json
import math
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
    ap.add_argument("--cold-iters", type=int, default=20,
                    help="extra decode calls each preceded by a 1 GiB write that evicts L2/MALL")
    ap.add_argument("--cpu-sample-seqs", type=int, default=16)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported in this build "
              f"(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import torch

    import paged_kv_cache_444_amd as pa
    from workloads import named_case

    print("bench: generating the 70B-shape batch-128 decode workload", file=sys.stderr, flush=True)
    case = named_case(2)
    d = case.decode
    Hq, Hkv, D, bs = case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    B = d.num_seqs
    max_len = d.max_seq_len

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    kc, vc = dev(case.key_cache), dev(case.value_cache)
    q = dev(d.query)
    bt = torch.from_numpy(d.block_tables).cuda()
    sl = torch.from_numpy(d.seq_lens).cuda()
    out = torch.empty_like(q)
    ws_bytes = pa.decode_workspace_bytes(B, Hq, D, max_len)
    ws = torch.empty(max(ws_bytes, 1), dtype=torch.uint8, device="cuda")
    scale = float(case.scale)

    def step():
        pa.decode(q, kc, vc, bt, sl, num_kv_heads=Hkv, block_size=bs, scale=scale,
                  max_seq_len=max_len, out=out, workspace=ws)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    pa.trace_enable(True)
    pa.trace_read("decode_partition")
    pa.trace_read("decode_merge")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.steps):
        step()
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    pa.trace_enable(False)
    n_part, ms_part = pa.trace_read("decode_partition")
    n_merge, ms_merge = pa.trace_read("decode_merge")

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    nbytes = decode_bytes(d.seq_lens, Hq, Hkv, D, bs)
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    part_ms = ms_part / max(n_part, 1)
    part_gbs = nbytes / (part_ms * 1e-3) / 1e9

    # Cold-cache variant: evict caches before each call; event-timed around the call only.
    cold_us = None
    if args.cold_iters > 0:
        flush = torch.empty(1 << 30, dtype=torch.uint8, device="cuda")
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        ts = []
        for _ in range(args.cold_iters):
            flush.fill_(1)
            e0.record()
            step()
            e1.record()
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)
        cold_us = float(np.median(ts))
        del flush

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(case, args.cpu_sample_seqs)

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
            "decode_partition_tokens": int(os.environ.get("PA_DECODE_PART", "512")),
        },
        "roofline": {
            "bound": "hbm", "kernel": "decode_partition", "achieved": round(part_gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(part_gbs / HBM_PEAK_GBS, 4),
            "traffic": None, "launch_us": round(part_ms * 1e3, 2),
            "merge_launch_us": round(ms_merge / max(n_merge, 1) * 1e3, 2),
        },
        "cold_cache_us_per_call": None if cold_us is None else round(cold_us, 2),
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def cpu_baseline(case, n_seqs):
    """Time the fp64 oracle on the first `n_seqs` sequences of the batch (all heads)."""
    from oracle import paged_attention as oracle

    d = case.decode
    seqs = list(range(min(n_seqs, d.num_seqs)))
    t0 = time.perf_counter()
    oracle.decode(d.query, case.key_cache, case.value_cache, d.block_tables, d.seq_lens,
                  case.num_kv_heads, case.head_dim, case.block_size, case.scale, seqs=seqs)
    dt = time.perf_counter() - t0
    nbytes = decode_bytes(d.seq_lens[seqs], case.num_q_heads, case.num_kv_heads, case.head_dim,
                          case.block_size)
    return {"value": round(nbytes / dt / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "seconds": round(dt, 3), "seqs_per_s": round(len(seqs) / dt, 3),
            "sample": f"first {len(seqs)} of {d.num_seqs} sequences, all 64 query heads, fp64 NumPy "
                      f"(gather + einsum, single-threaded)"}


if __name__ == "__main__":
    main()
