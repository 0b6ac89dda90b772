#!/usr/bin/env python3
"""Benchmark of one sparse MLA decode step on one MI355X (gfx950).

A step is the whole hot path over one batch: one sparse_mla_decode call of
libsmla.so, i.e. the split-K decode kernel and, when the list is split, the
log-sum-exp combine kernel.
Default workload: 32 query tokens x 64 heads, 512 of 32768 cache rows per
sequence (synthetic, seeded).

Inputs are resident in HBM before timing starts.  To keep each step reading
HBM rather than the 256 MB last-level cache, the timed loop rotates over R
copies of the inputs (distinct buffers, same contents) whose total footprint
exceeds 768 MB.  Warmup steps run first, untimed.  The timed region of K steps
is bracketed by synchronisations; HIP events on the launch stream at both ends
time the whole loop.  A second timed loop of K decode-kernel launches alone
gives that kernel's average duration for the roofline.

Prints one JSON line with queries*heads/s, effective KV GB/s, the roofline
object of the decode kernel (algorithmic KV bytes = 604 per kept row with fp32
group scales, 583 with UE8M0 scale bytes), and the fp64 CPU oracle timed on
the host as a baseline.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "sparse-MLA decode queries·heads/s + effective KV GB/s (% of MI355X roofline)"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E
BF16_PEAK_TFLOPS = 2500.0       # MI355X dense bf16/fp16 MFMA
# bytes of a kept row the decode must read: 448 fp8 codes + 7 group scales
# (fp32, or one byte each in the UE8M0 format) + 64 bf16 rope values
ROW_ALGO_BYTES = {0: 448 + 7 * 4 + 128, 1: 448 + 7 + 128}


def log(*a):
    print(*a, file=sys.stderr, flush=True)


COUNTER_SUMMARY = os.path.join(ROOT, "profiles", "decode_b32_h64_s32768_k512_kernel_stats.txt")
COUNTER_CONFIG = 3


def code_digest(source: str) -> str:
    """sha256[:16] of a C++ source with its // and /* */ comments and blank
    lines removed: it changes when the code does, not when a comment does."""
    source = re.sub(r"/\*.*?\*/", "", source, flags=re.S)
    lines = [re.sub(r"//.*$", "", ln).rstrip() for ln in source.splitlines()]
    return hashlib.sha256("\n".join(ln for ln in lines if ln.strip()).encode()).hexdigest()[:16]


def kernel_digest() -> str:
    """code_digest of the library's kernel sources and the compiler flags they
    are built with: what the machine code of the profiled kernels depends on."""
    from sparse_mla_decode_02_amd import build as hip_build
    csrc = os.path.join(ROOT, "sparse_mla_decode_02_amd", "csrc")
    text = "".join(open(os.path.join(csrc, f)).read() for f in sorted(os.listdir(csrc)) if f.endswith(".hip"))
    # the flags as a line of their own (not a comment, which code_digest drops)
    flags = hip_build.HIPCC_FLAGS + hip_build.VGPR_FORM + hip_build.PRELOAD + hip_build.SCHED_ILP + \
        hip_build.SCHED_CLAUSE
    return code_digest(text + "\nflags: " + " ".join(flags))


def counted_traffic(config, row_format):
    """HBM bytes per decode launch (FETCH_SIZE + WRITE_SIZE, calibrated against a
    plain device copy) from the committed rocprofv3 counter summary, when that
    summary was taken on this workload and on the current kernel source; None
    otherwise."""
    if config != COUNTER_CONFIG or row_format != 0 or not os.path.exists(COUNTER_SUMMARY):
        return None
    text = open(COUNTER_SUMMARY).read()
    digest = kernel_digest()
    m_src = re.search(r"code sha256\[:16\] = ([0-9a-f]{16})", text)
    m_dec = re.search(r"decode kernel(?: \([^)]*\))?: FETCH_SIZE .*?-> ([0-9.]+) MB per launch; WRITE_SIZE .*?-> ([0-9.]+) MB",
                      text)
    if not m_src or not m_dec or m_src.group(1) != digest:
        return None
    return (float(m_dec.group(1)) + float(m_dec.group(2))) * 1e6


# Positions of q, topk_idx and seqlens in the argument tuple of each C entry
# point that bench.py times (tests/test_bench_records.py checks them against
# include/smla.h).
ENTRY_ARG_POS = {
    "sparse_mla_decode": (0, 2, 3),
    "sparse_mla_decode_paged": (0, 3, 4),
    "sparse_mla_decode_single_launch": (0, 3, 4),
    "sparse_mla_decode_per_head": (0, 2, 3),
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=400)
    ap.add_argument("--warmup", type=int, default=40)
    ap.add_argument("--config", type=int, default=3, help="workload number 1..5 (default 3)")
    ap.add_argument("--num-splits", type=int, default=0, help="0 = library heuristic")
    ap.add_argument("--kernel", default="shared", choices=("shared", "per-head"),
                    help="shared: the decode path; per-head: the per-head SIMT ablation kernel")
    ap.add_argument("--single-launch", action="store_true",
                    help="time sparse_mla_decode_single_launch: split partials merged inside the decode kernel")
    ap.add_argument("--page-size", type=int, default=0,
                    help="0 = contiguous cache; else rows in a shuffled paged pool of this page size")
    ap.add_argument("--page-order", default="shuffled", choices=("shuffled", "sequential"),
                    help="pool pages in random order (default) or in sequence order")
    ap.add_argument("--row-format", type=int, default=0, choices=(0, 1),
                    help="cache rows: 0 = fp32 group scales (640 B), 1 = UE8M0 scale bytes (584 B)")
    ap.add_argument("--rotate", type=int, default=0, help="input copies (0 = auto, > 768 MB)")
    ap.add_argument("--cpu-seconds", type=float, default=10.0)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--warm", action="store_true", help="no rotation (last-level-cache warm)")
    ap.add_argument("--oracle-table", action="store_true",
                    help="host only: time the fp64 oracle on every workload (all threads; one thread "
                         "for workloads 1-3), median of 3 runs, and exit")
    ap.add_argument("--copy-calibration-mib", type=int, default=0,
                    help="run one plain device copy of this many MiB before timing (counter calibration)")
    return ap.parse_args()


def cpu_model() -> str:
    try:
        for ln in open("/proc/cpuinfo"):
            if ln.startswith("model name"):
                return ln.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def oracle_table(args):
    """The fp64 CPU oracle timed on every workload on this host: a reported
    baseline, not a target.  All threads (OpenMP default) for workloads 1-5,
    then one thread for workloads 1-3; each entry the median of 3 runs."""
    import oracle
    from workloads import build_host_cache, config_workload
    rows = []
    for threads, cfgs in ((0, (1, 2, 3, 4, 5)), (1, (1, 2, 3))):
        for c in cfgs:
            w = config_workload(c, row_format=args.row_format)
            hc = build_host_cache(w)
            times, used = [], 0
            for _ in range(3):
                t0 = time.perf_counter()
                _, _, used = oracle.decode_raw(w.q_bits, hc, w.kv_seq_stride, w.idx, w.seqlens, w.heads, w.scale,
                                               row_format=w.row_format, nthreads=threads)
                times.append(time.perf_counter() - t0)
            del hc
            t = sorted(times)[1]
            row = {"workload": w.name, "config_number": c, "threads": int(used), "median_s": t,
                   "queries_heads_per_s": w.batch * w.heads / t,
                   "kv_gbps": float(w.valid.sum()) * ROW_ALGO_BYTES[w.row_format] / t / 1e9}
            rows.append(row)
            log(f"oracle {w.name}: {used} threads, median {t * 1e3:.1f} ms, "
                f"{row['queries_heads_per_s']:.3g} q*h/s")
    print(json.dumps({"kind": "oracle timing", "cpu": cpu_model(), "nproc": os.cpu_count(),
                      "omp_num_threads": os.environ.get("OMP_NUM_THREADS"), "rows": rows}))


def main():
    args = parse()
    if args.oracle_table:
        oracle_table(args)
        return
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU only: the decode path shards by heads or sequences "
              "with no exchange, so multi-GPU runs are not part of this benchmark "
              "(use --gpus 1).", file=sys.stderr)
        sys.exit(2)

    import torch

    import sparse_mla_decode_02_amd as smla
    from workloads import config_workload, make_paged_layout, physical_rows

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.current_stream()

    t0 = time.time()
    w = config_workload(args.config, row_format=args.row_format)
    B, H, K = w.batch, w.heads, w.topk
    RB, fmt = w.row_bytes, w.row_format
    valid = w.valid
    n_rows = int(valid.sum())
    log(f"workload {w.name}: B={B} H={H} topk={K} stride={w.kv_seq_stride} kept rows={n_rows} "
        f"(generated in {time.time() - t0:.1f}s)")

    ns = smla.num_splits(B, H, K, args.num_splits, w.kv_seq_stride, fmt)
    chunk = smla.split_size(B, H, K, args.num_splits, w.kv_seq_stride, fmt)

    # ---- device inputs: R rotating copies
    b_i, j_i = np.nonzero(valid)
    paged = args.page_size > 0
    if paged:
        lay = make_paged_layout(w, args.page_size, seed=args.config, spare_pages=64,
                                shuffle=args.page_order == "shuffled")
        phys = physical_rows(w, lay)[b_i, j_i]
        assert (phys >= 0).all() and phys.max(initial=-1) < lay.num_pages * lay.page_size
        flat = torch.from_numpy(phys).to(dev)
        cache_rows = lay.num_pages * lay.page_size
        log(f"paged pool: page size {lay.page_size}, {lay.num_pages} pages, table {lay.block_table.shape}")
    else:
        flat = torch.from_numpy(b_i.astype(np.int64) * w.kv_seq_stride + w.idx[b_i, j_i]).to(dev)
        cache_rows = B * w.kv_seq_stride
    rows = torch.from_numpy(np.ascontiguousarray(w.rows[b_i, j_i])).to(dev)
    step_bytes = n_rows * RB + B * H * 512 * 2 * 2 + B * K * 4
    cache_bytes = cache_rows * RB
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
    bt0 = torch.from_numpy(lay.block_table).to(dev) if paged else None
    for r in range(R):
        cache = torch.full((cache_rows, RB), 0xFF, dtype=torch.uint8, device=dev)
        cache[flat] = rows
        sets.append((q0.clone(), cache, idx0.clone(), sl0.clone(), bt0.clone() if paged else None))
    out = torch.empty((B, H, 512), dtype=torch.bfloat16, device=dev)
    lse = torch.empty((B, H), dtype=torch.float32, device=dev)
    o_part = torch.empty((B, H, ns, 512), dtype=torch.float32, device=dev)
    lse_part = torch.empty((B, H, ns), dtype=torch.float32, device=dev)
    torch.cuda.synchronize()
    log(f"num_splits={ns} chunk={chunk} rotation R={R} ({R * step_bytes / 1e6:.0f} MB touched per "
        f"cycle, {R * cache_bytes / 1e9:.1f} GB allocated)")

    # Prebuilt C-ABI argument tuples per input copy, so that each timed launch
    # is a single ctypes call (the host must stay ahead of the GPU).
    import ctypes
    L = smla.lib()
    shape = smla.make_shape(B, H, K, args.num_splits, w.kv_seq_stride, fmt)
    pg = smla.make_paged(lay.page_size, lay.pages_per_seq, lay.num_pages) if paged else None
    hs = ctypes.c_void_p(stream.cuda_stream)
    P = lambda t: ctypes.c_void_p(t.data_ptr())
    dec_args, full_args = [], []
    ws = None
    need_ws = smla.workspace_bytes(B, H, K, args.num_splits, w.kv_seq_stride, fmt)
    if need_ws:
        ws = torch.empty(need_ws, dtype=torch.uint8, device=dev)
    wsp = P(ws) if ws is not None else None
    for q, cache, idx, sl, bt in sets:
        if paged:
            dec_args.append((P(q), P(cache), P(bt), P(idx), P(sl), ctypes.c_float(w.scale), ctypes.byref(shape),
                             ctypes.byref(pg), P(o_part), P(lse_part), hs))
            full_args.append((P(q), P(cache), P(bt), P(idx), P(sl), ctypes.c_float(w.scale), P(out), P(lse),
                              ctypes.byref(shape), ctypes.byref(pg), wsp, ctypes.c_size_t(need_ws), hs))
        else:
            dec_args.append((P(q), P(cache), P(idx), P(sl), ctypes.c_float(w.scale), ctypes.byref(shape),
                             P(o_part), P(lse_part), hs))
            full_args.append((P(q), P(cache), P(idx), P(sl), ctypes.c_float(w.scale), P(out), P(lse),
                              ctypes.byref(shape), wsp, ctypes.c_size_t(need_ws), hs))
    decode_fn = L.sparse_mla_decode_paged if paged else L.sparse_mla_decode
    partials_fn = L.sparse_mla_decode_partials_paged if paged else L.sparse_mla_decode_partials
    if args.kernel == "per-head":
        assert not paged, "the per-head ablation kernel reads a contiguous cache"
        ns = 1
        full_args = [(P(q), P(cache), P(idx), P(sl), ctypes.c_float(w.scale), P(out), P(lse), ctypes.byref(shape), hs)
                     for q, cache, idx, sl, _ in sets]
        decode_fn = L.sparse_mla_decode_per_head
    if args.single_launch:
        assert args.kernel == "shared", "the single launch is a form of the shared-read path"
        counters = torch.zeros(B * (H // 16), dtype=torch.int32, device=dev)   # arrival counters, left at zero
        full_args = [(P(q), P(cache), P(bt) if paged else None, P(idx), P(sl), ctypes.c_float(w.scale), P(out),
                      P(lse), ctypes.byref(shape), ctypes.byref(pg) if paged else None, wsp,
                      ctypes.c_size_t(need_ws), P(counters), hs) for q, cache, idx, sl, bt in sets]
        decode_fn = L.sparse_mla_decode_single_launch

    def step(i):
        """One whole step: decode kernel, then the combine kernel when split."""
        st = decode_fn(*full_args[i % R])
        assert st == 0, st

    def decode_only(i):
        """The decode kernel alone (split partials when the list is split; the
        whole step in the single launch)."""
        if ns == 1 or args.single_launch:
            st = decode_fn(*full_args[i % R])
        else:
            st = partials_fn(*dec_args[i % R])
        assert st == 0, st

    if args.copy_calibration_mib > 0:
        n = args.copy_calibration_mib << 20
        src_t = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst_t = torch.empty(n, dtype=torch.uint8, device=dev)
        torch.cuda.synchronize()
        dst_t.copy_(src_t)
        torch.cuda.synchronize()
        del src_t, dst_t
        log(f"calibration copy: {args.copy_calibration_mib} MiB read + written")

    # the rotation continues across the warmup and every timed loop, so that
    # no timed call reuses a copy touched less than R - 1 calls before
    rot = [0]

    def timed(fn, k):
        """k back-to-back calls bracketed by synchronisations; HIP events on the
        launch stream at both ends (no events between launches)."""
        a_ev = torch.cuda.Event(enable_timing=True)
        b_ev = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        w0 = time.perf_counter()
        i0 = rot[0]
        rot[0] += k
        a_ev.record(stream)
        for i in range(i0, i0 + k):
            fn(i)
        b_ev.record(stream)
        torch.cuda.synchronize()
        return a_ev.elapsed_time(b_ev) / k, (time.perf_counter() - w0) / k * 1e3

    # ---- warmup (untimed), on the first W copies of the rotation
    for i in range(args.warmup):
        step(i)
    rot[0] = args.warmup
    torch.cuda.synchronize()

    # ---- timed region: K whole steps (decode + combine), then K decode launches
    # alone for the decode kernel's own average duration
    ms_per_step, wall_ms = timed(step, args.steps)
    dec_ms, _ = timed(decode_only, args.steps)
    # secondary, labelled: the same inputs every step (last-level cache warm),
    # and each step's own duration (events around every step, rotated inputs)
    warm_ms, _ = timed(lambda i: step(0), args.steps)
    # KV cold, q / list / lengths warm: rotated caches, the first copy's other inputs
    # (the positions by entry point; checked on the host against the first copy
    # before any launch)
    qp, ip, sp = ENTRY_ARG_POS[decode_fn.__name__]
    assert full_args[0][qp].value == sets[0][0].data_ptr()
    assert full_args[0][ip].value == sets[0][2].data_ptr() and full_args[0][sp].value == sets[0][3].data_ptr()
    kvcold_args = []
    for a in full_args:
        a = list(a)
        a[qp], a[ip], a[sp] = P(sets[0][0]), P(sets[0][2]), P(sets[0][3])
        kvcold_args.append(tuple(a))
    kvcold_ms, _ = timed(lambda i: decode_fn(*kvcold_args[i % R]), args.steps)
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(args.steps + 1)]
    torch.cuda.synchronize()
    i0 = rot[0]
    rot[0] += args.steps
    evs[0].record(stream)
    for i in range(args.steps):
        step(i0 + i)
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    per_step = np.array([evs[i].elapsed_time(evs[i + 1]) * 1e3 for i in range(args.steps)])
    comb_ms = ms_per_step - dec_ms if ns > 1 else 0.0
    t_dec = dec_ms * 1e-3
    kv_bytes = ROW_ALGO_BYTES[fmt] * n_rows
    all_bytes = kv_bytes + B * H * 512 * 2 * 2 + B * H * 4 + B * K * 4 + B * 4
    kv_gbps = kv_bytes / t_dec / 1e9
    flops = 2048.0 * H * n_rows
    value = B * H / (ms_per_step * 1e-3)
    log(f"timed {args.steps} steps: {ms_per_step * 1e3:.2f} us/step (host wall {wall_ms * 1e3:.2f} us), "
        f"decode alone {dec_ms * 1e3:.2f} us/launch, combine ~{comb_ms * 1e3:.2f} us, KV {kv_gbps:.0f} GB/s")

    # ---- CPU baseline: the fp64 oracle on the host cores (bounded sample)
    cpu = None
    if not args.no_cpu_baseline:
        import oracle
        from workloads import build_host_cache
        hc = build_host_cache(w)
        reps, t_cpu, used = 0, 0.0, 0
        while t_cpu < args.cpu_seconds and reps < 1000:
            c0 = time.perf_counter()
            _, _, used = oracle.decode_raw(w.q_bits, hc, w.kv_seq_stride, w.idx, w.seqlens, H, w.scale,
                                           row_format=fmt)
            t_cpu += time.perf_counter() - c0
            reps += 1
        del hc
        cpu = {"value": B * H * reps / t_cpu, "unit": "queries·heads/s", "cores": int(used),
               "kind": "oracle", "cpu": cpu_model(), "nproc": os.cpu_count(),
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
                   "row_format": "ue8m0_scales_584B" if fmt == 1 else "fp32_scales_640B",
                   "cache": (f"paged, {args.page_size} rows per page, {args.page_order} pages" if paged
                             else "contiguous per sequence"),
                   "kernel": ("per-head SIMT ablation" if args.kernel == "per-head" else
                              "shared-read MFMA, single launch" if args.single_launch else "shared-read MFMA"),
                   "parallelism": "single-gpu"},
        "roofline": {"bound": "hbm", "achieved": kv_gbps, "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": kv_gbps / HBM_PEAK_GBPS,
                     "traffic": None if (paged or args.single_launch) else counted_traffic(args.config, fmt)},
        "cpu_baseline": cpu,
        "effective_kv_gbps": kv_gbps,
        "all_algorithmic_gbps": all_bytes / t_dec / 1e9,
        "decode_us": t_dec * 1e6,
        "step_us_percentiles": {"p10": float(np.percentile(per_step, 10)), "p50": float(np.median(per_step)),
                                "p90": float(np.percentile(per_step, 90)),
                                "note": "events around every step, rotated inputs"},
        "warm_step_us": warm_ms * 1e3,
        "kv_cold_q_warm_step_us": kvcold_ms * 1e3,
        "combine_us": comb_ms * 1e3,
        "mfma_tflops": flops / t_dec / 1e12,
        "mfma_frac": flops / t_dec / 1e12 / BF16_PEAK_TFLOPS,
        "precision": "fp8 e4m3fn + bf16 KV; QK bf16 MFMA, PV fp16 MFMA, fp32 accumulate; bf16 out",
        "timing": "HIP events on the launch stream around K back-to-back steps, then around K "
                  "decode-kernel launches alone; inputs rotated over R HBM-resident copies",
    }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
