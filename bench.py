#!/usr/bin/env python3
"""Benchmark of one sparse MLA decode step on one MI355X (gfx950).

A step is the whole hot path over one batch: the split-K decode kernel and,
when the list is split, the log-sum-exp combine kernel, both in libsmla.so.
Default workload: 32 query tokens x 64 heads, 512 of 32768 cache rows per
sequence (synthetic, seeded).

Inputs are resident in HBM before timing starts.  To keep each step reading
HBM rather than the 256 MB last-level cache, the timed loop rotates over R
copies of the inputs (distinct buffers, same contents) whose total footprint
exceeds 768 MB.  Warmup steps run first, untimed.  The timed region of K steps
is bracketed by synchronisations; HIP events on the launch stream time the
whole loop and every decode and combine launch inside it.

Prints one JSON line with queries*heads/s, effective KV GB/s, the roofline
object of the decode kernel (algorithmic KV bytes = 604 per kept row), and
the fp64 CPU oracle timed on the host as a baseline.
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

METRIC = "sparse-MLA decode queries·heads/s + effective KV GB/s (% of MI355X roofline)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16/fp16 MFMA
ROW_ALGO_BYTES = 604            # 448 fp8 + 7 fp32 scales + 64 bf16 rope per kept row


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", type=int, default=3, help="workload number 1..5 (default 3)")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = library heuristic")
    ap.add_argument("--rotate", type=int, default=0, help="input copies (0 = auto, > 768 MB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="no rotation (last-level-cache warm)")
    return ap.parse_args()


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path shards by heads or sequences "
              "with no exchange, so multi-GPU runs are not part of this benchmark "
              "(use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mla_decode_02_amd as smla
    from workloads import CONFIGS, ROW_BYTES, config_workload

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    t0 = time.time()
    w = config_workload(args.config)
    B, H, K = w.batch, w.heads, w.topk
    valid = w.valid
    n_rows = int(valid.sum())
    log(f"workload {w.name}: B={B} H={H} topk={K} stride={w.kv_seq_stride} kept rows={n_rows} "
        f"(generated in {time.time() - t0:.1f}s)")

    ns = smla.num_splits(B, H, K, args.num_splits, w.kv_seq_stride)
    chunk = smla.split_size(B, H, K, args.num_splits, w.kv_seq_stride)

    # ---- device inputs: R rotating copies
    b_i, j_i = np.nonzero(valid)
    flat = torch.from_numpy(b_i.astype(np.int64) * w.kv_seq_stride + w.idx[b_i, j_i]).to(dev)
    rows = torch.from_numpy(np.ascontiguousarray(w.rows[b_i, j_i])).to(dev)
    step_bytes = n_rows * ROW_BYTES + B * H * 512 * 2 * 2 + B * K * 4
    cache_bytes = B * w.kv_seq_stride * ROW_BYTES
    if args.warm:
        R = 1
    elif args.rotate > 0:
        R = args.rotate
    else:
        R = max(2, math.ceil(768e6 / step_bytes))
        R = min(R, 64, max(1, int(120e9 // cache_bytes)))
    sets = []
    q0 = torch.from_numpy(w.q_bits.view(np.int16)).to(dev).view(torch.bfloat16)
    idx0 = torch.from_numpy(w.idx).to(dev)
    sl0 = torch.from_numpy(w.seqlens).to(dev)
    for r in range(R):
        cache = torch.full((B, w.kv_seq_stride, ROW_BYTES), 0xFF, dtype=torch.uint8, device=dev)
        cache.view(-1, ROW_BYTES)[flat] = rows
        sets.append((q0.clone(), cache, idx0.clone(), sl0.clone()))
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    o_part = torch.empty((B, H, ns, 512), dtype=torch.float32, device=dev)
    lse_part = torch.empty((B, H, ns), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"num_splits={ns} chunk={chunk} rotation R={R} ({R * step_bytes / 1e6:.0f} MB touched per "
        f"cycle, {R * cache_bytes / 1e9:.1f} GB allocated)")

    def step(i):
        q, cache, idx, sl = sets[i % R]
        if ns == 1:
            smla.sparse_mla_decode(q, cache, idx, sl, w.scale, out, lse, num_splits=args.num_splits,
                                   kv_seq_stride=w.kv_seq_stride, stream=stream)
        else:
            smla.sparse_mla_decode_partials(q, cache, idx, sl, w.scale, o_part, lse_part,
                                            num_splits=args.num_splits,
                                            kv_seq_stride=w.kv_seq_stride, stream=stream)
            ev_mid[i].record(stream)
            smla.sparse_mla_combine(o_part, lse_part, out, lse, stream=stream)

    # ---- warmup (untimed)
    ev_mid = [torch.cuda.Event(enable_timing=True) for _ in range(max(args.warmup, args.steps))]
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    # ---- timed region: K steps
    ev_a = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    ev_b = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps)]
    start = torch.cuda.Event(enable_timing=True)
    end = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    wall0 = time.perf_counter()
    start.record(stream)
    for i in range(args.steps):
        ev_a[i].record(stream)
        step(i)
        ev_b[i].record(stream)
    end.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    total_ms = start.elapsed_time(end)
    ms_per_step = total_ms / args.steps
    step_ms = np.array([ev_a[i].elapsed_time(ev_b[i]) for i in range(args.steps)])
    if ns == 1:
        dec_ms = step_ms
        comb_ms = np.zeros_like(step_ms)
    else:
        dec_ms = np.array([ev_a[i].elapsed_time(ev_mid[i]) for i in range(args.steps)])
        comb_ms = np.array([ev_mid[i].elapsed_time(ev_b[i]) for i in range(args.steps)])
    t_dec = float(dec_ms.mean()) * 1e-3
    kv_bytes = ROW_ALGO_BYTES * n_rows
    all_bytes = kv_bytes + B * H * 512 * 2 * 2 + B * H * 4 + B * K * 4 + B * 4
    kv_gbps = kv_bytes / t_dec / 1e9
    flops = 2048.0 * H * n_rows
    value = B * H / (ms_per_step * 1e-3)
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.2f} us/step (wall {wall * 1e3 / args.steps:.2f} us), "
        f"decode {t_dec * 1e6:.2f} us (p10 {np.percentile(dec_ms, 10) * 1e3:.2f}, "
        f"p90 {np.percentile(dec_ms, 90) * 1e3:.2f}), combine {comb_ms.mean() * 1e3:.2f} us, "
        f"KV {kv_gbps:.0f} GB/s")

    # ---- CPU baseline: the fp64 oracle on the host cores (bounded sample)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from workloads import build_host_cache
        hc = build_host_cache(w)
        reps, t_cpu, used = 0, 0.0, 0
        while t_cpu < args.cpu_seconds and reps < 1000:
            c0 = time.perf_counter()
            _, _, used = oracle.decode_raw(w.q_bits, hc, w.kv_seq_stride, w.idx, w.seqlens, H, w.scale)
            t_cpu += time.perf_counter() - c0
            reps += 1
        del hc
        cpu = {"value": B * H * reps / t_cpu, "unit": "queries·heads/s", "cores": int(used),
               "kind": "oracle",
               "sample": f"{reps} full runs of the {w.name} workload ({B * H} query-heads each), "
                         f"{t_cpu:.1f} s, fp64 OpenMP over (b,h)"}
        log(f"cpu oracle: {cpu['value']:.3g} q*h/s on {used} threads ({reps} reps, {t_cpu:.1f}s)")

    res = {
        "metric": METRIC,
        "value": value,
        "unit": "queries·heads/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": w.name, "config_number": args.config, "batch": B, "heads": H,
                   "topk": K, "seq_len": int(w.kv_seq_stride), "kept_rows": n_rows,
                   "num_splits": ns, "split_size": chunk, "rotation": R,
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": kv_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": kv_gbps / HBM_PEAK_GBPS, "traffic": None},
        "cpu_baseline": cpu,
        "effective_kv_gbps": kv_gbps,
        "all_algorithmic_gbps": all_bytes / t_dec / 1e9,
        "decode_us": t_dec * 1e6,
        "decode_us_p10": float(np.percentile(dec_ms, 10)) * 1e3,
        "decode_us_p90": float(np.percentile(dec_ms, 90)) * 1e3,
        "combine_us": float(comb_ms.mean()) * 1e3,
        "mfma_tflops": flops / t_dec / 1e12,
        "mfma_frac": flops / t_dec / 1e12 / BF16_PEAK_TFLOPS,
        "precision": "fp8 e4m3fn + bf16 KV; QK bf16 MFMA, PV fp16 MFMA, fp32 accumulate; bf16 out",
        "timing": "HIP events on the launch stream; inputs rotated over R HBM-resident copies",
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
