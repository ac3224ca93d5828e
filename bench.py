"""Benchmark: paged decode attention at the Llama-3.3-70B shape, batch 128, on one MI355X.

One step = one pa_decode call over 128 sequences (64 query / 8 KV heads, head_dim 128, 16-token
blocks, lognormal context lengths with mean 1,500 and standard deviation 600 clipped to
[16, 8192]) whose K/V, queries and tables are already resident in HBM.  Consecutive steps cycle
through `--layers` distinct copies of the KV pools, as consecutive decode calls of a model touch
different layers' caches, so a step cannot be served from the 256 MB last-level cache that the
previous step filled.  Prints one JSON line.

  value        algorithmic bytes of one call / wall time per step (GB/s), K steps with nothing
               but the calls on the stream
  roofline     the dominant kernel (decode_kernel): algorithmic bytes per launch / its mean
               duration over the same K steps run again with HIP events recorded around every
               kernel launch (the events' marker packets add a few us per step, so this second
               pass is not the one `value` is taken from), against the 8 TB/s HBM peak
  call_us      per-call durations (events around each call on its stream): p10 / p50 / p90
  cpu_baseline the fp64 CPU oracle on the same batch, spread over the host's cores (a correctness
               tool, not an optimised CPU kernel), with every other workload under `per_config`
  paged_waste  share of allocated block slots the workloads leave empty (last blocks only), next
               to a contiguous 8,192-token reservation per sequence

  tp8_share    one GPU's share of the same batch at tensor parallelism 8 over KV heads (8 query
               heads on 1 KV head): call time, kernel roofline

  mixed_step   the chunked-prefill mixed step of the same model shape (one 512-token chunk over
               31,744 cached tokens, batched with 127 decode sequences): per-kernel times and the
               prefill kernel's MFMA roofline (causal FLOPs / its event-timed duration against the
               2.5 PFLOP/s dense bf16 peak)

  cow_step     a copy-on-write step of rollouts sharing a 4,100-token prompt (8 prompts x 16
               candidates): block copies, the new tokens' reshape and the decode, per kernel

`--mode copy` instead times a plain device-to-device copy of a known size: the calibration run for
the FETCH_SIZE / WRITE_SIZE hardware counters.  `--mode mixed` / `--mode cow` run only that step.
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
MFMA_BF16_PEAK_TFLOPS = 2500.0
# Untimed calls before the secondary fields (FP8 cache, TP=8 share) are timed: the default run's
# warmup, whatever --warmup gives the headline step.
SECONDARY_WARMUP = 100
METRIC = "pa_decode achieved HBM GB/s (% of peak) + seqs/s, 70B-shape B=128"


def decode_bytes(seq_lens, Hq, Hkv, D, bs):
    """Algorithmic HBM bytes of one decode call: each sequence's K and V once, its query read and
    output written once, its used block-table entries and its length."""
    L = np.asarray(seq_lens, dtype=np.int64)
    kv = int((L * Hkv * D * 2 * 2).sum())
    qo = len(L) * 2 * Hq * D * 2
    tables = int(((L + bs - 1) // bs).sum()) * 4 + len(L) * 4
    return kv + qo + tables


def prefill_flops(query_start_loc, seq_lens, Hq, D):
    """Causal attention FLOPs of a prefill chunk: one multiply-add (2 FLOPs) per head dimension for
    q·k and one for p·v, per visible (query row, key) pair and head:
    4 * D * Hq * (sum over rows of the keys each row sees)."""
    qsl = np.asarray(query_start_loc, dtype=np.int64)
    total = 0
    for i, L in enumerate(np.asarray(seq_lens, dtype=np.int64)):
        q = int(qsl[i + 1] - qsl[i])
        ctx = int(L) - q
        total += q * ctx + q * (q + 1) // 2
    return 4 * D * Hq * total


def reshape_bytes(T, Hkv, D):
    """Algorithmic bytes of reshape_and_cache: K and V rows read and written, slots read."""
    return 4 * T * Hkv * D * 2 + 8 * T


def measured_traffic(kernel):
    """HBM bytes per launch of `kernel` measured with FETCH_SIZE / WRITE_SIZE (profiles/traffic.json),
    or None when the kernel's sources changed since the counters were taken."""
    import hashlib

    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    rec = json.load(open(path)).get(kernel)
    if not rec:
        return None
    h = hashlib.sha256()
    for src in rec["sources"]:
        with open(os.path.join(ROOT, src), "rb") as f:
            h.update(f.read())
    return rec["hbm_bytes_per_launch"] if h.hexdigest() == rec["sources_sha256"] else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=100)
    ap.add_argument("--layers", type=int, default=4,
                    help="distinct KV pool copies cycled through by consecutive steps")
    ap.add_argument("--warm-steps", type=int, default=50,
                    help="extra steps on one pool (cache-warm), reported for context")
    ap.add_argument("--cpu-runs", type=int, default=3,
                    help="timed runs of the CPU oracle per workload (the median is reported)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--dist-steps", type=int, default=100,
                    help="calls timed one by one for the p10/p50/p90 of the call duration")
    ap.add_argument("--no-tp-share", action="store_true",
                    help="skip the tensor-parallel share (8 query heads on 1 KV head)")
    ap.add_argument("--mode", choices=["decode", "copy", "mixed", "cow", "prefix", "configs"],
                    default="decode")
    ap.add_argument("--mixed-steps", type=int, default=30)
    ap.add_argument("--mixed-warmup", type=int, default=60)
    ap.add_argument("--mixed-order", choices=["decode-first", "prefill-first"], default="decode-first",
                    help="which half of the overlapped mixed step is launched first")
    ap.add_argument("--no-mixed", action="store_true", help="skip the mixed-step measurement")
    ap.add_argument("--no-cow", action="store_true", help="skip the copy-on-write step measurement")
    ap.add_argument("--no-fp8", action="store_true", help="skip the FP8-cache decode measurement")
    ap.add_argument("--no-prefix", action="store_true",
                    help="skip the prefix-shared (plain vs cascade decode) measurement")
    ap.add_argument("--cow-steps", type=int, default=50)
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
              f"(the library's path runs on a single GPU: run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    if not args.no_cpu_baseline and args.mode == "decode":
        # The CPU baseline's worker processes fork from a server started before this process
        # touches the GPU.
        from oracle import pool

        pool.start()

    import torch

    if args.mode == "copy":
        run_copy(args)
        return
    if args.mode == "mixed":
        print(json.dumps(run_mixed(args)), flush=True)
        return
    if args.mode == "cow":
        print(json.dumps(run_cow(args)), flush=True)
        return
    if args.mode == "prefix":
        print(json.dumps(run_prefix_shared(args)), flush=True)
        return
    if args.mode == "configs":
        print(json.dumps(run_configs(args)), flush=True)
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

    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    log(f"timed {args.steps} steps")

    pa.trace_enable(True)
    for name in ("decode_partition", "decode_merge"):
        pa.trace_read(name)
    torch.cuda.synchronize()
    t2 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    t3 = time.perf_counter()
    n_main, ms_main = pa.trace_read("decode_partition")
    n_merge, ms_merge = pa.trace_read("decode_merge")
    pa.trace_enable(False)
    log(f"timed {args.steps} steps with per-launch events")

    # Per-call distribution: events around each call on its stream.
    ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
          for _ in range(args.dist_steps)]
    for i, (a, b) in enumerate(ev):
        a.record()
        step(i)
        b.record()
    torch.cuda.synchronize()
    call_us = np.array([a.elapsed_time(b) * 1e3 for a, b in ev])

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

    ms_per_step = (t1 - t0) * 1e3 / args.steps
    nbytes = decode_bytes(d.seq_lens, Hq, Hkv, D, bs)
    gbs = nbytes / (ms_per_step * 1e-3) / 1e9
    main_ms = ms_main / max(n_main, 1)
    main_gbs = nbytes / (main_ms * 1e-3) / 1e9

    fp8 = None
    if not args.no_fp8:
        fp8 = run_fp8_decode(args, case, pools, q, bt, sl, out, ws, ms_per_step, main_ms)
    n_pools = len(pools)
    # The measured read ceiling comes after the decode timing: run first, its 25 passes over
    # 4 GiB left the decode 1.5 % slower (alternating fresh processes on one box).
    ceiling = stream_read_ceiling()
    log(f"stream-read ceiling {ceiling['gbs']} GB/s")
    tp = None
    if not args.no_tp_share:
        del pools, kc0, vc0
        pools = None
        torch.cuda.empty_cache()
        tp = run_tp_share(args)
    mixed = None
    if not args.no_mixed:
        pools = kc0 = vc0 = None
        torch.cuda.empty_cache()
        mixed = run_mixed(args)
    cow = None
    if not args.no_cow:
        cow = run_cow(args)
    prefix = None
    if not args.no_prefix:
        prefix = run_prefix_shared(args)

    cpu = None
    if not args.no_cpu_baseline:
        log("timing the CPU oracle on every workload")
        cpu = cpu_baseline(args)

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
            "pool_copies_cycled": n_pools,
            "decode_workers": int(os.environ.get("PA_DECODE_WORKERS", "0")) or "default",
            "decode_prefetch": int(os.environ.get("PA_DECODE_PREFETCH", "1")),
            "decode_static_q10": int(os.environ.get("PA_DECODE_STATIC_Q10", "1024")),
            "decode_chunk_steps": int(os.environ.get("PA_DECODE_CHUNK", "4")),
            "decode_step": "vector" if os.environ.get("PA_DECODE_MFMA") == "0" else "matrix cores",
        },
        "roofline": {
            "bound": "hbm", "kernel": "decode_kernel", "achieved": round(main_gbs, 1),
            "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(main_gbs / HBM_PEAK_GBS, 4),
            "traffic": measured_traffic("decode_kernel"), "launch_us": round(main_ms * 1e3, 2),
            "merge_launch_us": round(ms_merge / max(n_merge, 1) * 1e3, 2),
            "ms_per_step_with_events": round((t3 - t2) * 1e3 / args.steps, 5),
        },
        "call_us": {"p10": round(float(np.percentile(call_us, 10)), 2),
                    "p50": round(float(np.percentile(call_us, 50)), 2),
                    "p90": round(float(np.percentile(call_us, 90)), 2),
                    "mean": round(float(call_us.mean()), 2), "calls": int(call_us.size),
                    "how": "events recorded around each call on its stream, pools cycled"},
        "warm_single_pool_us_per_step": None if warm_us is None else round(warm_us, 2),
        "stream_read_ceiling": dict(ceiling,
                                    decode_kernel_frac=round(main_gbs / ceiling["gbs"], 4),
                                    decode_call_frac=round(gbs / ceiling["gbs"], 4)),
        "tp8_share": tp,
        "paged_waste": paged_waste_report(),
        "fp8_decode": fp8,
        "mixed_step": mixed,
        "cow_step": cow,
        "prefix_shared": prefix,
        "cpu_baseline": cpu,
    }
    print(json.dumps(rec), flush=True)


def stream_read_ceiling(gib=4, reps=20):
    """The measured HBM read ceiling: the library's plain streaming-read kernel (every byte of a
    `gib` GiB buffer once, 16-byte non-temporal loads) timed with events on its stream."""
    import torch

    import paged_kv_cache_444_amd as pa

    buf = torch.empty(gib << 30, dtype=torch.uint8, device="cuda")
    sink = pa.stream_read(buf)
    for _ in range(5):
        pa.stream_read(buf, sink)
    torch.cuda.synchronize()
    pa.trace_enable(True)
    pa.trace_read("stream_read")
    for _ in range(reps):
        pa.stream_read(buf, sink)
    torch.cuda.synchronize()
    n, ms = pa.trace_read("stream_read")
    pa.trace_enable(False)
    del buf, sink
    torch.cuda.empty_cache()
    us = ms / n * 1e3
    return {"kernel": "stream_read_kernel", "bytes": gib << 30, "us": round(us, 1),
            "gbs": round((gib << 30) / (us * 1e-6) / 1e9, 1)}


def fp8_decode_bytes(seq_lens, Hq, Hkv, D, bs):
    """Algorithmic bytes of one decode call over an FP8 cache: K and V one byte per element, the
    bf16 query and output, the used table entries and the lengths."""
    L = np.asarray(seq_lens, dtype=np.int64)
    return int((L * Hkv * D * 2).sum()) + len(L) * 2 * Hq * D * 2 + \
        int(((L + bs - 1) // bs).sum()) * 4 + len(L) * 4


def run_fp8_decode(args, case, pools, q, bt, sl, out, ws, bf16_ms, bf16_kernel_ms):
    """The same batch over an FP8 E4M3 cache (per-tensor scales 6/448 for K, 5.5/448 for V): the
    bf16 pools are quantised on the device once (torch's float8_e4m3fn conversion after a clamp to
    +-448; a synthetic-input step, outside the timed region), then timed like the bf16 decode."""
    import torch

    import paged_kv_cache_444_amd as pa

    d = case.decode
    Hq, Hkv, D, bs = case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    ks, vs = 6.0 / 448.0, 5.5 / 448.0

    def q8(t, s):
        return (t.float() / s).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)

    pools8 = [(q8(kc, ks), q8(vc, vs)) for kc, vc in pools]
    torch.cuda.synchronize()

    def step(i):
        kc8, vc8 = pools8[i % len(pools8)]
        pa.decode_fp8(q, kc8, vc8, bt, sl, num_kv_heads=Hkv, block_size=bs, k_scale=ks, v_scale=vs,
                      scale=float(case.scale), max_seq_len=d.max_seq_len, out=out, workspace=ws)

    # The FP8 pools are fresh allocations: the secondary fields warm up as the default run does
    # (at least 100 untimed calls), whatever --warmup gives the headline step.
    log("FP8 cache: warmup")
    for i in range(max(args.warmup, SECONDARY_WARMUP)):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    pa.trace_enable(True)
    pa.trace_read("decode_partition")
    pa.trace_read("decode_merge")
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    n_main, ms_main = pa.trace_read("decode_partition")
    n_merge, ms_merge = pa.trace_read("decode_merge")
    pa.trace_enable(False)
    kms = ms_main / max(n_main, 1)
    nbytes = fp8_decode_bytes(d.seq_lens, Hq, Hkv, D, bs)
    gbs = nbytes / (ms * 1e-3) / 1e9
    kgbs = nbytes / (kms * 1e-3) / 1e9
    log(f"FP8 cache: {ms * 1e3:.1f} us per call, kernel {kms * 1e3:.1f} us")
    del pools8
    return {
        "kv_dtype": "fp8_e4m3", "k_scale": ks, "v_scale": vs, "algorithmic_bytes": nbytes,
        "warmup": max(args.warmup, SECONDARY_WARMUP), "steps": args.steps,
        "ms_per_step": round(ms, 5), "gbs": round(gbs, 1),
        "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
        "seqs_per_s": round(d.num_seqs / (ms * 1e-3), 1),
        "speedup_vs_bf16_call": round(bf16_ms / ms, 3),
        "roofline": {"bound": "hbm", "kernel": "decode_kernel (fp8)", "achieved": round(kgbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(kgbs / HBM_PEAK_GBS, 4),
                     "traffic": measured_traffic("decode_kernel_fp8"),
                     "launch_us": round(kms * 1e3, 2),
                     "merge_launch_us": round(ms_merge / max(n_merge, 1) * 1e3, 2),
                     "speedup_vs_bf16_kernel": round(bf16_kernel_ms / kms, 3)},
        "prefetch_depth": int(os.environ.get("PA_DECODE_PREFETCH_FP8", "1")),
    }


def run_mixed(args):
    """Chunked-prefill mixed step of the 70B shape: reshape of the chunk's K/V, the prefill chunk,
    then decode of the 127 other sequences, all resident in HBM, on one stream."""
    import torch

    import paged_kv_cache_444_amd as pa
    from workloads import named_case

    log("generating the mixed chunked-prefill workload")
    case = named_case(4)
    Hq, Hkv, D, bs = case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    pf, dc, rs = case.prefill, case.decode, case.reshape

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    kc, vc = dev(case.key_cache), dev(case.value_cache)
    rk, rv, slots = dev(rs.key), dev(rs.value), torch.from_numpy(rs.slot_mapping).cuda()
    pq, pbt = dev(pf.query), torch.from_numpy(pf.block_tables).cuda()
    pqsl, psl = torch.from_numpy(pf.query_start_loc).cuda(), torch.from_numpy(pf.seq_lens).cuda()
    dq, dbt, dsl = dev(dc.query), torch.from_numpy(dc.block_tables).cuda(), torch.from_numpy(dc.seq_lens).cuda()
    pout, dout = torch.empty_like(pq), torch.empty_like(dq)
    pws = torch.zeros(max(pa.prefill_workspace_bytes(pf.num_seqs, pf.total_q, pf.max_q_len, Hq, Hkv, D,
                                                     pf.max_seq_len), 1), dtype=torch.uint8, device="cuda")
    dws = torch.zeros(max(pa.decode_workspace_bytes(dc.num_seqs, Hq, Hkv, D, dc.max_seq_len), 1),
                      dtype=torch.uint8, device="cuda")
    scale = float(case.scale)

    side = torch.cuda.Stream()
    main_stream = torch.cuda.current_stream()

    def do_prefill():
        pa.prefill_chunk(pq, kc, vc, pbt, pqsl, psl, num_kv_heads=Hkv, block_size=bs,
                         max_q_len=pf.max_q_len, max_seq_len=pf.max_seq_len, scale=scale, out=pout,
                         workspace=pws)

    def do_decode():
        pa.decode(dq, kc, vc, dbt, dsl, num_kv_heads=Hkv, block_size=bs, scale=scale,
                  max_seq_len=dc.max_seq_len, out=dout, workspace=dws)

    def serial_step():
        pa.reshape_and_cache(rk, rv, kc, vc, slots, num_kv_heads=Hkv, head_dim=D, block_size=bs)
        do_prefill()
        do_decode()

    pre_args = dict(query=pq, key_cache=kc, value_cache=vc, block_tables=pbt, query_start_loc=pqsl,
                    seq_lens=psl, num_kv_heads=Hkv, block_size=bs, max_q_len=pf.max_q_len,
                    max_seq_len=pf.max_seq_len, scale=scale, out=pout, workspace=pws)
    dec_args = dict(query=dq, key_cache=kc, value_cache=vc, block_tables=dbt, seq_lens=dsl,
                    num_kv_heads=Hkv, block_size=bs, scale=scale, max_seq_len=dc.max_seq_len,
                    out=dout, workspace=dws)

    def overlapped_step():
        # The new tokens are written first; then decode runs on a second stream beside the
        # prefill chunk, and the step ends when both have finished.
        pa.reshape_and_cache(rk, rv, kc, vc, slots, num_kv_heads=Hkv, head_dim=D, block_size=bs)
        if args.mixed_order == "decode-first":
            pa.mixed_step(pre_args, dec_args, side_stream=side)
            return
        side.wait_stream(main_stream)
        with torch.cuda.stream(side):
            do_prefill()
        do_decode()
        main_stream.wait_stream(side)

    names = ("reshape_and_cache", "prefill_chunk", "prefill_merge", "decode_partition", "decode_merge")

    def timed(step):
        # The matrix cores' clock ramps up over the first few tens of milliseconds of this load.
        for _ in range(args.mixed_warmup):
            step()
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for _ in range(args.mixed_steps):
            step()
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e3 / args.mixed_steps

    ms_step = timed(serial_step)
    ms_overlap = timed(overlapped_step)
    ms_step2 = timed(serial_step)
    # Per-kernel durations from a second pass with events around every launch.
    pa.trace_enable(True)
    for n in names:
        pa.trace_read(n)
    for _ in range(args.mixed_steps):
        serial_step()
    torch.cuda.synchronize()
    per = {}
    for n in names:
        k, ms = pa.trace_read(n)
        per[n] = round(ms / k * 1e3, 2) if k else None
    pa.trace_enable(False)
    # The same step over an FP8 cache (pools converted on the device with torch's float8_e4m3fn
    # cast after a clamp to +-448: input preparation, outside the timed region).
    ks, vs = 6.0 / 448.0, 5.5 / 448.0
    kc8 = (kc.float() / ks).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    vc8 = (vc.float() / vs).clamp_(-448.0, 448.0).to(torch.float8_e4m3fn).view(torch.uint8)
    pre8 = dict(pre_args, key_cache=kc8, value_cache=vc8, k_scale=ks, v_scale=vs)
    dec8 = dict(dec_args, key_cache=kc8, value_cache=vc8, k_scale=ks, v_scale=vs)

    def fp8_serial():
        pa.reshape_and_cache_fp8(rk, rv, kc8, vc8, slots, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                                 k_scale=ks, v_scale=vs)
        pa.prefill_chunk_fp8(**pre8)
        pa.decode_fp8(**dec8)

    def fp8_overlapped():
        pa.reshape_and_cache_fp8(rk, rv, kc8, vc8, slots, num_kv_heads=Hkv, head_dim=D, block_size=bs,
                                 k_scale=ks, v_scale=vs)
        pa.mixed_step(pre8, dec8, side_stream=side, fp8=True)

    ms8_serial = timed(fp8_serial)
    ms8_overlap = timed(fp8_overlapped)
    pa.trace_enable(True)
    for n in names:
        pa.trace_read(n)
    for _ in range(args.mixed_steps):
        fp8_serial()
    torch.cuda.synchronize()
    per8 = {}
    for n in names:
        k, ms = pa.trace_read(n)
        per8[n] = round(ms / k * 1e3, 2) if k else None
    pa.trace_enable(False)
    del kc8, vc8

    flops = prefill_flops(pf.query_start_loc, pf.seq_lens, Hq, D)
    pre_us = per["prefill_chunk"]
    tflops = flops / (pre_us * 1e-6) / 1e12
    dbytes = decode_bytes(dc.seq_lens, Hq, Hkv, D, bs)
    rbytes = reshape_bytes(len(rs.slot_mapping), Hkv, D)
    log(f"mixed step {ms_step * 1e3:.1f} us serial ({ms_step2 * 1e3:.1f} us again), "
        f"{ms_overlap * 1e3:.1f} us with decode beside the prefill chunk")
    return {
        "workload": case.name, "us_per_step": round(ms_step * 1e3, 2), "steps": args.mixed_steps,
        "warmup": args.mixed_warmup,
        "us_per_step_serial_again": round(ms_step2 * 1e3, 2),
        "us_per_step_overlapped": round(ms_overlap * 1e3, 2), "overlap_order": args.mixed_order,
        "kernel_us": per,
        "prefill_roofline": {"bound": "mfma", "kernel": "prefill_chunk",
                             "achieved": round(tflops, 1), "peak": MFMA_BF16_PEAK_TFLOPS,
                             "unit": "TFLOP/s", "frac": round(tflops / MFMA_BF16_PEAK_TFLOPS, 4),
                             "flops_per_launch": flops},
        "decode_gbs": round(dbytes / (per["decode_partition"] * 1e-6) / 1e9, 1),
        "fp8": {"us_per_step_serial": round(ms8_serial * 1e3, 2),
                "us_per_step_overlapped": round(ms8_overlap * 1e3, 2), "kernel_us": per8,
                "prefill_tflops": round(flops / (per8["prefill_chunk"] * 1e-6) / 1e12, 1)},
        "reshape_gbs": round(rbytes / (per["reshape_and_cache"] * 1e-6) / 1e9, 1),
        "reshape_bytes": rbytes, "decode_bytes": dbytes,
    }


def run_cow(args):
    """Copy-on-write step of rollouts at the 70B shape: 8 prompts x 16 candidates share a
    4,100-token prompt whose last block holds 4 tokens.  Every candidate writes its first token at
    position 4,100; all but the last holder of each group first copy that block (120 copies), then
    the 128 tokens are written and the 128 sequences decoded.  Repeating the step rewrites the same
    bytes, so every repetition does the same work."""
    import torch

    import paged_kv_cache_444_amd as pa
    from workloads import build_cow_case

    log("generating the copy-on-write rollout step")
    case, copies = build_cow_case("cow_rollouts_8x16_prompt4100", 8, 16, 4100, 64, 8, 128, 16,
                                  (444, 64))
    Hq, Hkv, D, bs = case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    d, r = case.decode, case.reshape

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    kc, vc = dev(case.key_cache), dev(case.value_cache)
    cm = torch.from_numpy(copies).cuda()
    rk, rv, slots = dev(r.key), dev(r.value), torch.from_numpy(r.slot_mapping).cuda()
    q, bt, sl = dev(d.query), torch.from_numpy(d.block_tables).cuda(), torch.from_numpy(d.seq_lens).cuda()
    out = torch.empty_like(q)
    ws = torch.zeros(max(pa.decode_workspace_bytes(d.num_seqs, Hq, Hkv, D, d.max_seq_len), 1),
                     dtype=torch.uint8, device="cuda")
    kw = dict(num_kv_heads=Hkv, head_dim=D, block_size=bs)

    def step():
        pa.copy_blocks(kc, vc, cm, **kw)
        pa.reshape_and_cache(rk, rv, kc, vc, slots, **kw)
        pa.decode(q, kc, vc, bt, sl, num_kv_heads=Hkv, block_size=bs, scale=float(case.scale),
                  max_seq_len=d.max_seq_len, out=out, workspace=ws)

    for _ in range(20):
        step()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(args.cow_steps):
        step()
    torch.cuda.synchronize()
    us_step = (time.perf_counter() - t0) * 1e6 / args.cow_steps
    names = ("copy_blocks", "reshape_and_cache", "decode_partition", "decode_merge")
    pa.trace_enable(True)
    for n in names:
        pa.trace_read(n)
    for _ in range(args.cow_steps):
        step()
    torch.cuda.synchronize()
    per = {}
    for n in names:
        k, ms = pa.trace_read(n)
        per[n] = round(ms / k * 1e3, 2) if k else None
    pa.trace_enable(False)
    block_bytes = Hkv * bs * D * 2
    cbytes = 4 * len(copies) * block_bytes  # K and V blocks, each read once and written once
    log(f"copy-on-write step {us_step:.1f} us")
    # Larger copies on the same pools: a copy-on-write step moves too few blocks to reach the HBM
    # rate, so the rate at 1,200 and 6,000 random pairs is reported beside it.
    sweep = {}
    rng = np.random.default_rng(7)
    n_pool = case.num_blocks - 1  # the last block is the poison block
    for pairs in (1200, 6000):
        if 2 * pairs > n_pool:
            continue
        ids = rng.permutation(n_pool)
        m = torch.from_numpy(np.stack([ids[:pairs], ids[pairs:2 * pairs]], 1).astype(np.int64)).cuda()
        for _ in range(5):
            pa.copy_blocks(kc, vc, m, **kw)
        pa.trace_enable(True)
        pa.trace_read("copy_blocks")
        for _ in range(20):
            pa.copy_blocks(kc, vc, m, **kw)
        torch.cuda.synchronize()
        k, ms = pa.trace_read("copy_blocks")
        pa.trace_enable(False)
        us = ms / k * 1e3
        sweep[str(pairs)] = {"us": round(us, 2), "gbs": round(4 * pairs * block_bytes / us / 1e3, 1)}
    return {
        "workload": case.name, "us_per_step": round(us_step, 2), "steps": args.cow_steps,
        "copies": len(copies), "new_tokens": len(r.slot_mapping), "kernel_us": per,
        "copy_blocks_bytes": cbytes,
        "copy_blocks_gbs": round(cbytes / (per["copy_blocks"] * 1e-6) / 1e9, 1),
        "copy_blocks_random_pairs": sweep,
        "decode_logical_gbs": round(decode_bytes(d.seq_lens, Hq, Hkv, D, bs)
                                    / (per["decode_partition"] * 1e-6) / 1e9, 1),
    }


def run_prefix_shared(args):
    """Prefix-shared rollouts at the 70B shape (8 prompts x 16 candidates sharing a 4,096-token
    prompt's blocks, private tails of 0..1,024 tokens, one new token each): plain decode against
    the cascade decode that reads each shared prompt once per group.  Rates are given on the
    logical bytes (every sequence's K/V) and on the unique bytes (each physical block once)."""
    import torch

    import paged_kv_cache_444_amd as pa
    from workloads import named_case

    log("generating the prefix-shared rollout workload")
    case = named_case(5)
    Hq, Hkv, D, bs = case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
    d, r = case.decode, case.reshape

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    kc, vc = dev(case.key_cache), dev(case.value_cache)
    pa.reshape_and_cache(dev(r.key), dev(r.value), kc, vc, torch.from_numpy(r.slot_mapping).cuda(),
                         num_kv_heads=Hkv, head_dim=D, block_size=bs)
    # Distinct pool copies cycled by consecutive calls, so no call finds the previous call's blocks
    # in the last-level cache (each copy is 427 MB of K and V).
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(args.layers - 1)]
    q, bt, sl = dev(d.query), torch.from_numpy(d.block_tables).cuda(), torch.from_numpy(d.seq_lens).cuda()
    gs = torch.arange(0, d.num_seqs + 1, 16, dtype=torch.int32, device="cuda")
    out = torch.empty_like(q)
    ws = torch.zeros(max(pa.decode_workspace_bytes(d.num_seqs, Hq, Hkv, D, d.max_seq_len), 1),
                     dtype=torch.uint8, device="cuda")
    cws = torch.zeros(max(pa.decode_cascade_workspace_bytes(d.num_seqs, 8, 16, Hq, Hkv, D, 4096), 1),
                      dtype=torch.uint8, device="cuda")
    kw = dict(num_kv_heads=Hkv, block_size=bs, scale=float(case.scale), max_seq_len=d.max_seq_len,
              out=out)

    def plain(i):
        k, v = pools[i % len(pools)]
        pa.decode(q, k, v, bt, sl, workspace=ws, **kw)

    pl = torch.full((d.num_seqs,), 4096, dtype=torch.int32, device="cuda")

    def cascade(i):
        k, v = pools[i % len(pools)]
        pa.decode_cascade(q, k, v, bt, sl, gs, pl, max_prefix_len=4096, max_group_size=16,
                          workspace=cws, **kw)

    def timed(fn):
        for i in range(20):
            fn(i)
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        for i in range(args.cow_steps):
            fn(i)
        torch.cuda.synchronize()
        return (time.perf_counter() - t0) * 1e6 / args.cow_steps

    us_plain, us_cascade = timed(plain), timed(cascade)
    us_plain2, us_cascade2 = timed(plain), timed(cascade)
    names = ("prefill_chunk", "decode_partition", "cascade_merge")
    pa.trace_enable(True)
    for n in names:
        pa.trace_read(n)
    for i in range(args.cow_steps):
        cascade(i)
    torch.cuda.synchronize()
    per = {}
    for n in names:
        k, ms = pa.trace_read(n)
        per[n] = round(ms / k * 1e3, 2) if k else None
    pa.trace_enable(False)
    logical = decode_bytes(d.seq_lens, Hq, Hkv, D, bs)
    used = np.unique(np.concatenate([d.block_tables[i, :(int(L) + bs - 1) // bs]
                                     for i, L in enumerate(d.seq_lens)]))
    unique = int(used.size) * Hkv * bs * D * 2 * 2 + d.num_seqs * 2 * Hq * D * 2
    best_p, best_c = min(us_plain, us_plain2), min(us_cascade, us_cascade2)
    log(f"prefix-shared: plain decode {best_p:.1f} us, cascade {best_c:.1f} us")
    return {
        "workload": case.name, "logical_bytes": logical, "unique_bytes": unique,
        "plain_us": [round(us_plain, 2), round(us_plain2, 2)],
        "cascade_us": [round(us_cascade, 2), round(us_cascade2, 2)],
        "pool_copies_cycled": len(pools),
        "cascade_speedup": round(best_p / best_c, 3),
        "cascade_kernel_us": per,
        "cascade_unique_gbs": round(unique / (best_c * 1e-6) / 1e9, 1),
        "cascade_logical_gbs": round(logical / (best_c * 1e-6) / 1e9, 1),
        "plain_logical_gbs": round(logical / (best_p * 1e-6) / 1e9, 1),
    }


def run_configs(args):
    """Decode kernel time on each named decode workload (tiny; 70B shape; wide-head; prefix-shared,
    plain decode), one pool per workload, after its new tokens are written: per-call kernel
    time from HIP events and algorithmic GB/s.  Context for the parity workloads, not the metric."""
    import torch

    import paged_kv_cache_444_amd as pa
    from workloads import named_case

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    res = {}
    for cfg in (1, 2, 3, 5):
        case = named_case(cfg)
        Hq, Hkv, D, bs = case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size
        d = case.decode
        log(f"configs: {case.name}")
        kc, vc = dev(case.key_cache), dev(case.value_cache)
        if case.reshape is not None:
            r = case.reshape
            pa.reshape_and_cache(dev(r.key), dev(r.value), kc, vc,
                                 torch.from_numpy(r.slot_mapping).cuda(), num_kv_heads=Hkv,
                                 head_dim=D, block_size=bs)
        q, bt, sl = dev(d.query), torch.from_numpy(d.block_tables).cuda(), torch.from_numpy(d.seq_lens).cuda()
        out = torch.empty_like(q)
        ws = torch.zeros(max(pa.decode_workspace_bytes(d.num_seqs, Hq, Hkv, D, d.max_seq_len), 1),
                         dtype=torch.uint8, device="cuda")

        def step():
            pa.decode(q, kc, vc, bt, sl, num_kv_heads=Hkv, block_size=bs, scale=float(case.scale),
                      max_seq_len=d.max_seq_len, out=out, workspace=ws)

        for _ in range(30):
            step()
        torch.cuda.synchronize()
        pa.trace_enable(True)
        pa.trace_read("decode_partition")
        pa.trace_read("decode_merge")
        for _ in range(50):
            step()
        torch.cuda.synchronize()
        n, ms = pa.trace_read("decode_partition")
        nm, msm = pa.trace_read("decode_merge")
        pa.trace_enable(False)
        us = ms / n * 1e3
        nbytes = decode_bytes(d.seq_lens, Hq, Hkv, D, bs)
        res[case.name] = {"kernel_us": round(us, 2), "merge_us": round(msm / max(nm, 1) * 1e3, 2),
                          "algorithmic_bytes": nbytes,
                          "kernel_gbs": round(nbytes / (us * 1e-6) / 1e9, 1),
                          "pct_of_hbm_peak": round(100 * nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBS, 2)}
        del kc, vc
        torch.cuda.empty_cache()
    return {"mode": "configs", "note": "one pool per workload (no cycling of copies)",
            "workloads": res}


def paged_waste_report():
    """Share of the allocated block slots that the workloads' sequences leave empty.  Blocks are
    taken as tokens arrive, so only each sequence's last block is partly empty; shared prompt
    blocks are counted once.  Next to it, the share of a contiguous reservation of 8,192 tokens
    per sequence that goes unused (the pages' fragmentation comparison)."""
    from workloads import NAMED_CASES

    out = {}
    for cfg, make in NAMED_CASES.items():
        spec = make()
        bs = spec.block_size
        lens = [int(x) for x in (spec.decode_lens or [])]
        lens += [int(c) + int(q) for c, q in (spec.prefill or [])]
        used = sum(lens)
        slots = sum(-(-L // bs) * bs for L in lens)
        for members, shared in (spec.share_groups or []):
            # every member after the first reuses the group's shared blocks
            used -= (len(members) - 1) * shared
            slots -= (len(members) - 1) * shared
        out[spec.name] = {"paged_waste_pct": round(100.0 * (1.0 - used / slots), 3),
                          "contiguous_8192_waste_pct":
                              round(100.0 * (1.0 - sum(lens) / (8192.0 * len(lens))), 1)
                              if max(lens) <= 8192 else None,
                          "tokens": used, "slots": slots, "block_size": bs}
    return out


def run_tp_share(args, tp=8, copies=8):
    """One GPU's share of the 70B-shaped batch-128 decode at tensor parallelism `tp` over KV
    heads: the same lengths, 64/tp query heads on 8/tp KV heads.  `copies` pool copies are cycled
    (1/tp of the bytes per call: more copies keep the last-level cache cold)."""
    import torch

    import paged_kv_cache_444_amd as pa
    from workloads import tp_share_case

    log(f"generating the TP={tp} share of the 70B-shaped decode")
    case = tp_share_case(tp)
    d = case.decode
    Hq, Hkv, D, bs = case.num_q_heads, case.num_kv_heads, case.head_dim, case.block_size

    def dev(a):
        return torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).cuda().view(torch.bfloat16)

    kc, vc = dev(case.key_cache), dev(case.value_cache)
    pools = [(kc, vc)] + [(kc.clone(), vc.clone()) for _ in range(copies - 1)]
    q, out = dev(d.query), None
    bt, sl = torch.from_numpy(d.block_tables).cuda(), torch.from_numpy(d.seq_lens).cuda()
    out = torch.empty_like(q)
    ws = torch.zeros(pa.decode_workspace_bytes(d.num_seqs, Hq, Hkv, D, d.max_seq_len),
                     dtype=torch.uint8, device="cuda")

    def step(i):
        k, v = pools[i % len(pools)]
        pa.decode(q, k, v, bt, sl, num_kv_heads=Hkv, block_size=bs, scale=float(case.scale),
                  max_seq_len=d.max_seq_len, out=out, workspace=ws)

    for i in range(max(args.warmup, SECONDARY_WARMUP)):
        step(i)
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) * 1e3 / args.steps
    pa.trace_enable(True)
    pa.trace_read("decode_partition")
    pa.trace_read("decode_merge")
    for i in range(args.steps):
        step(i)
    torch.cuda.synchronize()
    n_main, ms_main = pa.trace_read("decode_partition")
    n_merge, ms_merge = pa.trace_read("decode_merge")
    pa.trace_enable(False)
    kms = ms_main / max(n_main, 1)
    nbytes = decode_bytes(d.seq_lens, Hq, Hkv, D, bs)
    gbs, kgbs = nbytes / (ms * 1e-3) / 1e9, nbytes / (kms * 1e-3) / 1e9
    log(f"TP={tp} share: {ms * 1e3:.1f} us per call, kernel {kms * 1e3:.1f} us")
    del pools, kc, vc
    torch.cuda.empty_cache()
    return {"workload": case.name, "num_q_heads": Hq, "num_kv_heads": Hkv,
            "algorithmic_bytes": nbytes, "pool_copies_cycled": copies,
            "warmup": max(args.warmup, SECONDARY_WARMUP), "steps": args.steps,
            "us_per_call": round(ms * 1e3, 2), "gbs": round(gbs, 1),
            "pct_of_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2),
            "seqs_per_s": round(d.num_seqs / (ms * 1e-3), 1),
            "roofline": {"bound": "hbm", "kernel": "decode_kernel", "achieved": round(kgbs, 1),
                         "peak": HBM_PEAK_GBS, "unit": "GB/s",
                         "frac": round(kgbs / HBM_PEAK_GBS, 4), "launch_us": round(kms * 1e3, 2),
                         "merge_launch_us": round(ms_merge / max(n_merge, 1) * 1e3, 2)}}


def cpu_baseline(args):
    """The fp64 oracle (gather + attention, NumPy) on every workload, spread over the host's
    cores: each worker process runs the unchanged oracle on a share of the sequences (or of the
    chunk's query rows).  Input generation, the oracle's reshape of the step's new tokens and
    writing the pools for the workers are outside the timed region.  Median of --cpu-runs runs
    (one if a run exceeds 60 s)."""
    from oracle import paged_attention as oracle
    from oracle import pool
    from workloads import named_case

    pool.warm_up()
    cores = pool.workers()

    def timed(fn):
        runs = []
        while len(runs) < max(args.cpu_runs, 1):
            t0 = time.perf_counter()
            fn()
            runs.append(time.perf_counter() - t0)
            if runs[-1] > 60:
                break
        return float(np.median(runs)), len(runs)

    per = {}
    for cfg in (1, 2, 3, 4, 5):
        case = named_case(cfg)
        kc, vc = case.key_cache, case.value_cache
        if case.reshape is not None:
            r = case.reshape
            kc, vc = oracle.reshape_and_cache(kc, vc, r.key, r.value, r.slot_mapping,
                                              case.num_kv_heads, case.head_dim, case.block_size)
        d = case.decode
        sc = dict(num_kv_heads=case.num_kv_heads, head_dim=case.head_dim,
                  block_size=case.block_size, scale=case.scale)
        st = pool.Staged(dict(query=d.query, key_cache=kc, value_cache=vc,
                              block_tables=d.block_tables, seq_lens=d.seq_lens))
        try:
            sec, n = timed(lambda: st.run("decode", sc, "seqs", range(d.num_seqs)))
        finally:
            st.remove()
        nbytes = decode_bytes(d.seq_lens, case.num_q_heads, case.num_kv_heads, case.head_dim,
                              case.block_size)
        per[case.name] = {"seconds": round(sec, 4), "runs": n, "gbs": round(nbytes / sec / 1e9, 4),
                          "seqs_per_s": round(d.num_seqs / sec, 2),
                          "sample": f"decode of all {d.num_seqs} sequences"}
        if case.prefill is not None:
            # Two rows of every 16-token query tile (its first and last): a bounded sample.
            p = case.prefill
            rows = sorted({r for t in range(0, p.total_q, 16)
                           for r in (t, min(t + 15, p.total_q - 1))})
            stp = pool.Staged(dict(query=p.query, key_cache=kc, value_cache=vc,
                                   block_tables=p.block_tables, query_start_loc=p.query_start_loc,
                                   seq_lens=p.seq_lens))
            try:
                psec, pn = timed(lambda: stp.run("prefill_chunk", sc, "rows", rows))
            finally:
                stp.remove()
            ctx = int(p.seq_lens[0]) - p.total_q  # one sequence's chunk
            flops = 4 * case.head_dim * case.num_q_heads * sum(ctx + r + 1 for r in rows)
            per[case.name + " (prefill chunk)"] = {
                "seconds": round(psec, 4), "runs": pn,
                "tflops": round(flops / psec / 1e12, 6),
                "sample": f"{len(rows)} of {p.total_q} query rows (the first and last of every "
                          f"16-row tile), all {case.num_q_heads} heads"}
        del case, kc, vc
    head = per["llama70b_decode_b128"]
    try:
        import platform

        cpu_model = platform.processor() or platform.machine()
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        cpu_model = None
    return {"value": head["gbs"], "unit": "GB/s", "cores": cores, "kind": "oracle",
            "host_cores_available": len(os.sched_getaffinity(0)), "cpu_model": cpu_model,
            "seconds_per_call": head["seconds"], "seqs_per_s": head["seqs_per_s"],
            "sample": f"the whole 128-sequence batch, {cores} worker processes each running the "
                      f"fp64 NumPy oracle (gather + einsum, one thread each) on a share of the "
                      f"sequences; median of {head['runs']} runs",
            "per_config": per}


if __name__ == "__main__":
    main()
