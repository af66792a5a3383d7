#!/usr/bin/env python3
"""Benchmark of the selected-index NoPE MLA paged decode on one MI355X.

One step = one dsa_decode_launch (one kernel: selection normalisation, page
translation, gather, attention and the merge of split chunks) over one batch
of synthetic decode input, with every input already resident in HBM. The default workload is the long-context
decode share: 128 rows x 64 local heads, kv_lora_rank 512, 2048 selected ids
per row out of a 131072-token context, pages drawn from one 24 GiB FP8 pool.
Steps cycle through several independently drawn selection batches (and query
batches) so the gathered rows are not served from the 256 MiB last-level cache
by the previous step.

Prints one JSON line (rank 0) with the throughput in selected tokens/s, the
roofline of the decode kernel (gathered FP8 bytes / its HIP-event-timed
duration against 8 TB/s), the MFMA utilisation, and the CPU oracle timed on
the same workload on this host's cores.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, published
BF16_DENSE_TFLOPS = 2500.0      # MI355X dense bf16 MFMA, published


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    # ~50 ms of launches: the GPU's clocks take some tens of milliseconds of
    # load to settle (the first 200 launches run 10-20 % slower)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--workload", default="long",
                    choices=["glm", "long", "verify", "ragged", "latent_write"],
                    help="decode workload, or latent_write: the cache writer alone")
    ap.add_argument("--writer-rows", type=int, default=65536,
                    help="latent_write: rows written per launch")
    ap.add_argument("--sets", type=int, default=4,
                    help="distinct input batches cycled through")
    ap.add_argument("--cpu-rows", type=int, default=64,
                    help="rows of the workload the CPU oracle is timed on, on all its "
                         "threads (1/32 of them on one thread; 0: skip)")
    ap.add_argument("--calib-copy-mib", type=int, default=0,
                    help="also run one plain device copy of this many MiB "
                         "(reference dispatch for HBM counter calibration)")
    ap.add_argument("--flush-mib", type=int, default=0,
                    help="cold runs: sweep this many MiB (>= 512 evicts the 256 MiB "
                         "last-level cache) before every timed decode launch and time each "
                         "launch with its own event pair (reported as 'cold'; a kernel trace "
                         "gives the exact durations)")
    ap.add_argument("--flush-kind", choices=["read", "write"], default="read",
                    help="cold runs: the sweep reads the buffer (the caches hold clean lines "
                         "afterwards) or writes it (they hold dirty lines, which the decode's "
                         "own reads then push out to HBM)")
    ap.add_argument("--chunk-tokens", type=int, default=0)
    ap.add_argument("--layout", type=int, default=0, choices=[0, 1, 2, 3],
                    help="head blocks: 0 the planner's choice, 1 blocks of 32 heads, "
                         "2 blocks of 16, 3 blocks of 64")
    ap.add_argument("--rope-tail", action="store_true",
                    help="576-byte tokens: the latent plus a 64-byte rope tail (q 576 wide, "
                         "scores over 576, values over 512); no CPU baseline")
    ap.add_argument("--merge-in-kernel", action="store_true",
                    help="split rows merged by their last chunk inside the decode "
                         "kernel instead of by the combine kernel")
    ap.add_argument("--rows-per-sequence", type=int, default=-1,
                    help="decode_k rows per sequence co-scheduled on one XCD "
                         "(-1: the workload's own, 4 for verify, else 1)")
    return ap.parse_args()


def main():
    args = parse()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print(json.dumps({"error": "this decode path is built and measured on one GPU; "
                          "runs on more than one GPU are not part of it: rows shard "
                          "across GPUs with no exchange, heads shard with one "
                          "all-reduce after o_absorb", "n_gpus": args.gpus}))
        sys.exit(2)

    if args.workload == "latent_write":
        bench_latent_write(args)
        return

    import numpy as np
    import torch

    import sparse_attention_decode_row_amd as dsa
    import workloads as WL

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    name = args.workload
    t0 = time.time()

    base = WL.make(name, with_pool=False)
    R, H, D, W = base.rows, base.heads, base.D, base.width
    rope = 64 if args.rope_tail else 0
    TB = D + rope                                     # bytes per cached token
    if rope:
        import dataclasses
        import math
        base = dataclasses.replace(base, rope=rope, cache_stride_bytes=base.block_size * TB,
                                   sm_scale=1.0 / math.sqrt(TB))
        args.cpu_rows = 0
    pool = WL.device_pool(base.num_pages, base.block_size, TB, base.sigma,
                          base.k_scale, seed=base.seed)
    bt = torch.from_numpy(base.block_tables).to(dev)
    sl = torch.from_numpy(base.seq_lens).to(dev)
    batches = []
    uniq_per_step = []
    union_per_step = []
    rows_per_seq = (args.rows_per_sequence if args.rows_per_sequence >= 0
                    else (4 if name == "verify" else 1))
    for s in range(args.sets):
        wl = base if s == 0 else WL.make(name, sel_seed=s, with_pool=False)
        qb = np.random.default_rng([base.seed, 100 + s]).standard_normal((R, H, TB), dtype=np.float32)
        q = torch.from_numpy(WL.bf16_bits_from_f32(qb).view(np.int16)).to(dev).view(torch.bfloat16)
        sel = torch.from_numpy(wl.sel).to(dev)
        batches.append((q, sel))
        n = 0
        sets = []
        for r in range(R):
            row = wl.sel[r]
            sets.append(np.unique(row[(row >= 0) & (row < wl.seq_lens[r])]))
            n += int(sets[-1].size)
        uniq_per_step.append(n)
        # decode_k rows of one sequence: the union of their selections is what
        # the sequence needs from memory once
        k = max(rows_per_seq, 1)
        union_per_step.append(sum(int(np.unique(np.concatenate(sets[i:i + k])).size)
                                  for i in range(0, R, k)))
    out = torch.empty((R, H, D), dtype=torch.bfloat16, device=dev)
    # the verify workload holds 4 consecutive decode_k rows per sequence
    plan = dsa.Plan(num_rows=R, num_q_heads=H, kv_lora_rank=D,
                    block_size=base.block_size, index_kpool=base.kpool, sel_width=W,
                    block_table_stride=base.bt_stride, max_seq_len=base.max_seq_len,
                    sm_scale=base.sm_scale, cache_stride_bytes=base.cache_stride_bytes,
                    chunk_tokens=args.chunk_tokens, layout=args.layout,
                    merge_in_kernel=args.merge_in_kernel,
                    qk_rope_dim=rope, rows_per_sequence=rows_per_seq, device=0)
    ws = plan.new_workspace(0)
    info = plan.info()
    stream = torch.cuda.current_stream()
    sptr = int(stream.cuda_stream)
    print(f"[bench] {name}: rows {R} heads {H} D {D} W {W} pool "
          f"{base.pool_bytes / 2**30:.1f} GiB, plan {info}, setup {time.time() - t0:.1f}s",
          file=sys.stderr, flush=True)

    def step(i):
        q, sel = batches[i % args.sets]
        plan.launch(q, pool, pool, bt, sl, sel, base.k_scale, base.v_scale, out, ws,
                    stream=sptr)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()

    if args.calib_copy_mib:
        calibration_copy(args.calib_copy_mib)

    # The timed region is K launches back to back on the launch stream,
    # bracketed by one pair of HIP events (a pair around every launch would
    # itself cost ~12 us per step: each event record is a barrier packet).
    # One decode launch per step, so the kernel's average launch duration is
    # the region's event time over K.
    K = args.steps
    ev0 = torch.cuda.Event(enable_timing=True)
    ev1 = torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    t_start = time.perf_counter()
    ev0.record(stream)
    for i in range(K):
        step(args.warmup + i)
    ev1.record(stream)
    torch.cuda.synchronize()
    t_end = time.perf_counter()
    wall_ms = (t_end - t_start) * 1e3
    event_ms = ev0.elapsed_time(ev1)
    ms_per_step = wall_ms / K

    tokens = float(np.mean([uniq_per_step[(args.warmup + i) % args.sets] for i in range(K)]))
    value = tokens / (ms_per_step / 1e3)
    kern_ms = event_ms / K
    gathered_bytes = tokens * TB                     # FP8 token bytes per launch
    flops = 2.0 * H * (TB + D) * tokens              # QK^T over TB + PV over D
    achieved_gbps = gathered_bytes / (kern_ms / 1e3) / 1e9
    tflops = flops / (kern_ms / 1e3) / 1e12

    result = {
        "metric": "selected tokens/s per decode step (achieved HBM GB/s & MFMA util of the decode kernel alongside)",
        "value": value,
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8",
        "data": "synthetic",
        "config": {
            "workload": f"{name}: {R} rows x {H} heads, kv_lora_rank {D}"
                        + (f" + {rope}-byte rope tail" if rope else "")
                        + f", {W} selected ids "
                        f"per row of a {int(base.max_seq_len)}-token context, block_size "
                        f"{base.block_size}, FP8 E4M3 pool {base.pool_bytes / 2**30:.1f} GiB",
            "rows": R, "heads": H, "kv_lora_rank": D, "sel_width": W,
            "seq_len": int(base.max_seq_len), "block_size": base.block_size,
            "selected_tokens_per_step": tokens, "input_batches_cycled": args.sets,
            "plan": info,
        },
        "us_per_step": ms_per_step * 1e3,
        "us_per_step_gpu_events": event_ms * 1e3 / K,
        "kernel_us": {"dsa_decode_kernel": kern_ms * 1e3},
        "kernel_us_source": "HIP events around the timed region on the launch stream, / steps",
        "arithmetic": "FP8 E4M3 matrix-core products with fp32 accumulation; bf16 q "
                      "enters exactly as two FP8 terms, softmax weights as two FP8 terms "
                      "(relative error <= 2^-9); output bf16",
        "roofline": {
            "bound": "hbm",
            "kernel": "dsa_decode_kernel",
            "achieved": achieved_gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": achieved_gbps / HBM_PEAK_GBPS,
            "traffic": None,
            "algorithmic_bytes_per_launch": gathered_bytes,
        },
        # algorithmic flops; each is issued as two FP8 MFMA flops, so against
        # the 5.0 PFLOP/s FP8 peak the pipe utilisation is the same fraction
        "mfma": {"achieved": tflops, "peak": BF16_DENSE_TFLOPS, "unit": "TFLOP/s",
                 "frac": tflops / BF16_DENSE_TFLOPS, "flops_per_launch": flops,
                 "fp8_issued_flops_per_launch": 2 * flops, "fp8_peak": 5000.0},
    }

    if rows_per_seq > 1:
        utok = float(np.mean([union_per_step[(args.warmup + i) % args.sets] for i in range(K)]))
        ub = utok * TB
        result["union"] = {
            "rows_per_sequence": rows_per_seq, "tokens_per_step": utok, "gathered_bytes": ub,
            "achieved": ub / (kern_ms / 1e3) / 1e9, "unit": "GB/s",
            "frac": ub / (kern_ms / 1e3) / 1e9 / HBM_PEAK_GBPS,
            "note": "the distinct tokens each sequence's rows select, fetched once per "
                    "sequence: the bytes the method needs from memory"}
    if args.flush_mib:
        result["cold"] = cold_run(args, step, stream, D, TB, H, uniq_per_step)
    measured = None if rope else measured_traffic(name, rows_per_sequence=rows_per_seq)
    if measured is not None:
        result["roofline"]["traffic"] = measured
        result["roofline"]["traffic_unit"] = ("bytes per launch, rocprofv3 FETCH_SIZE + WRITE_SIZE "
                                              "scaled by a 256 MiB copy's readings")
    if args.cpu_rows > 0:
        result["cpu_baseline"] = cpu_baseline(base, pool, batches[0], args.cpu_rows)
    print(json.dumps(result), flush=True)


def cold_run(args, step, stream, D, TB, H, uniq_per_step):
    """Decode launches with the caches flushed before each: a sweep over
    args.flush_mib MiB (a reduction that reads it, or a fill that writes it),
    then the launch between its own event pair."""
    import numpy as np
    import torch
    flush = torch.ones(args.flush_mib << 17, dtype=torch.int64, device=stream.device)
    sink = torch.zeros(1, dtype=torch.int64, device=stream.device)
    n = min(args.steps, 200)
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n)]
    torch.cuda.synchronize()
    for i in range(n):
        if args.flush_kind == "read":
            torch.sum(flush, dim=0, keepdim=True, out=sink)
        else:
            flush.fill_(i)
        evs[i][0].record(stream)
        step(i)
        evs[i][1].record(stream)
    torch.cuda.synchronize()
    us = np.array([a.elapsed_time(b) * 1e3 for a, b in evs])
    tokens = float(np.mean([uniq_per_step[i % args.sets] for i in range(n)]))
    med = float(np.median(us))
    return {"flush_mib": args.flush_mib, "flush_kind": args.flush_kind, "launches": n,
            "kernel_us_median_events": med, "kernel_us_mean_events": float(us.mean()),
            "roofline_frac": tokens * TB / (med / 1e6) / 1e9 / HBM_PEAK_GBPS,
            "note": "each launch timed by its own event pair after a cache-flushing "
                    "sweep; an event pair adds a few microseconds, so a kernel trace's "
                    "durations are the precise cold figure"}


def calibration_copy(mib):
    """Reference dispatch for counter calibration: reads and writes exactly
    `mib` MiB once each."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda").fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    dst.copy_(src)
    torch.cuda.synchronize()
    print(f"[bench] calibration copy of {n} bytes done", file=sys.stderr, flush=True)


def measured_traffic(workload, kernel="dsa_decode_kernel", source="kernels.hip",
                     rows_per_sequence=None):
    """HBM bytes per launch from the committed counter summary of this
    kernel and workload, or None when there is none, the kernel source has
    changed since the counters were taken, or they were taken with another
    rows_per_sequence."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{kernel}_{workload}_hbm_counters.json")
    src = os.path.join(ROOT, "sparse_attention_decode_row_amd", "csrc", source)
    if not os.path.exists(path):
        return None
    with open(path) as f:
        rec = json.load(f)
    with open(src, "rb") as f:
        sha = hashlib.sha256(f.read()).hexdigest()
    if rec.get("kernel_source_sha256") != sha or rec.get("workload") != workload:
        return None
    if rows_per_sequence is not None and rec.get("rows_per_sequence", 1) != rows_per_sequence:
        return None
    return float(rec["traffic_bytes_per_launch"])


def cpu_baseline(wl, pool_dev, batch, nrows):
    """The CPU oracle, as it stands, on the first rows of the first batch
    (all heads, the full selection of each row): one warm-up run, then the
    median of 3 timed runs on every thread the oracle uses (the first
    `nrows` rows), and the same on one thread (a smaller sample of rows)."""
    import statistics

    import numpy as np
    import torch

    import oracle
    import workloads as WL

    rows = list(range(min(nrows, wl.rows)))
    rows_1t = rows[:max(1, len(rows) // 32)]
    assert wl.cache_stride_bytes == wl.block_size * wl.D
    # Pages the sample touches, renumbered compactly into a host pool that is
    # zero (untouched, never faulted in) except for the selected latent rows,
    # which are gathered on the GPU and copied over.
    pages = WL.pages_of_rows(wl, rows)
    remap = np.zeros(wl.num_pages, dtype=np.int64)
    remap[pages] = np.arange(pages.size, dtype=np.int64)
    bt = remap[wl.block_tables[rows]].astype(np.int32)
    src_rows, dst_rows = [], []
    for i, r in enumerate(rows):
        ids = np.unique(wl.sel[r][(wl.sel[r] >= 0) & (wl.sel[r] < wl.seq_lens[r])])
        page = wl.block_tables[r if wl.bt_stride else 0][ids // wl.block_size].astype(np.int64)
        slot = (ids % wl.block_size).astype(np.int64)
        src_rows.append(page * wl.block_size + slot)
        dst_rows.append(remap[page] * wl.block_size + slot)
    src_rows = np.concatenate(src_rows)
    dst_rows = np.concatenate(dst_rows)
    idx = torch.from_numpy(src_rows).to(pool_dev.device)
    got = pool_dev.view(-1, wl.D).index_select(0, idx).cpu().numpy()
    sub = np.zeros((pages.size * wl.block_size, wl.D), dtype=np.uint8)
    sub[dst_rows] = got
    sub = sub.ravel()
    q_all = batch[0].view(torch.int16).cpu().numpy().view(np.uint16)
    sel_all, sl_all = wl.sel, wl.seq_lens

    def tokens_of(rs):
        return sum(int(np.unique(sel_all[r][(sel_all[r] >= 0) & (sel_all[r] < sl_all[r])]).size)
                   for r in rs)

    def run(rs, threads):
        k = len(rs)
        t = time.perf_counter()
        oracle.decode(q_all[rs], sub, None, bt[:k], sl_all[rs], sel_all[rs],
                      block_size=wl.block_size, bt_stride=wl.bt_stride,
                      cache_stride_bytes=wl.cache_stride_bytes, sm_scale=wl.sm_scale,
                      k_scale=wl.k_scale, v_scale=wl.v_scale, num_threads=threads)
        return time.perf_counter() - t

    threads = oracle.max_threads()
    run(rows[:max(1, len(rows) // 8)], threads)                  # warm-up
    times = [run(rows, threads) for _ in range(3)]
    times_1t = [run(rows_1t, 1) for _ in range(3)]
    dt, dt1 = statistics.median(times), statistics.median(times_1t)
    tokens, tokens_1t = tokens_of(rows), tokens_of(rows_1t)
    return {"value": tokens / dt, "unit": "tokens/s", "cores": threads, "kind": "oracle",
            "sample": f"{len(rows)} of {wl.rows} rows of the same workload (all "
                      f"{wl.heads} heads, {tokens} selected tokens), float64 C oracle, "
                      f"median of 3 runs after one warm-up: "
                      f"{', '.join(f'{x:.2f}' for x in times)} s",
            "one_thread": {"value": tokens_1t / dt1, "unit": "tokens/s",
                           "sample": f"{len(rows_1t)} rows ({tokens_1t} selected tokens), "
                                     f"median of 3: {', '.join(f'{x:.2f}' for x in times_1t)} s"},
            "nproc": os.cpu_count(),
            "sched_affinity": len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else None}


def bench_latent_write(args):
    """The cache writer alone: N bf16 kv_a rows of kv_lora_rank 512, RMSNorm
    x weight / kv_scale, FP8 E4M3 into distinct random slots of a paged pool
    (block_size 64). HBM-bound: per row it reads 2*D bytes and writes D bytes
    (plus its 8-byte slot); the weight (2*D bytes) is read once per launch.
    Input sets are cycled so that the bytes touched over a cycle exceed the
    GPU's 256 MiB last-level cache."""
    import math

    import numpy as np
    import torch

    import sparse_attention_decode_row_amd as dsa

    assert torch.cuda.is_available(), "bench.py needs a GPU"
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    D, B, N = 512, 64, args.writer_rows
    eps, kv_scale = 1e-6, 0.02
    per_set = N * (3 * D + 8)
    sets = min(64, max(args.sets, math.ceil(512 * 2**20 / per_set)))
    slots_total = sets * N
    pages = (slots_total + B - 1) // B
    gen = torch.Generator(device=dev)
    gen.manual_seed(20240)
    pool = torch.zeros(pages * B * D, dtype=torch.uint8, device=dev)
    weight = (0.5 + torch.rand(D, generator=gen, device=dev)).to(torch.bfloat16)
    # every set writes its own rows to its own slots: a random permutation of
    # the pool's slots, dealt out N at a time
    perm = torch.randperm(pages * B, generator=gen, device=dev)[:slots_total]
    batches = []
    for s in range(sets):
        kv = torch.randn((N, D), generator=gen, device=dev).to(torch.bfloat16)
        batches.append((kv, perm[s * N:(s + 1) * N].contiguous()))
    stream = torch.cuda.current_stream()
    sptr = int(stream.cuda_stream)
    print(f"[bench] latent_write: {N} rows x {D}, {sets} input sets, pool "
          f"{pool.numel() / 2**20:.0f} MiB", file=sys.stderr, flush=True)

    def step(i, n=N):
        kv, sl = batches[i % sets]
        dsa.latent_write(kv[:n], weight, sl[:n], pool, block_size=B, rms_eps=eps,
                         inv_kv_scale=1.0 / kv_scale, stream=sptr)

    def region(K, first, n=N):
        ev0 = torch.cuda.Event(enable_timing=True)
        ev1 = torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        t = time.perf_counter()
        ev0.record(stream)
        for i in range(K):
            step(first + i, n)
        ev1.record(stream)
        torch.cuda.synchronize()
        return (time.perf_counter() - t) * 1e3, ev0.elapsed_time(ev1)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    if args.calib_copy_mib:
        calibration_copy(args.calib_copy_mib)
    K = args.steps
    wall_ms, event_ms = region(K, args.warmup)
    ms_per_step = wall_ms / K
    kern_ms = event_ms / K
    # one decode step's worth of new tokens (one per row of the long-context
    # batch): launch-bound, reported beside the bulk figure
    _, small_ms = region(K, 0, n=128)

    alg = N * (3 * D + 8) + 2 * D
    gbps = alg / (kern_ms / 1e3) / 1e9
    result = {
        "metric": "latent rows written to the FP8 paged cache per second",
        "value": N / (ms_per_step / 1e3),
        "unit": "rows/s",
        "n_gpus": 1,
        "steps": K,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {
            "workload": f"latent_write: {N} bf16 rows of kv_lora_rank {D} -> FP8 E4M3 "
                        f"into random distinct slots of a {pool.numel() / 2**20:.0f} MiB "
                        f"paged pool (block_size {B}), {sets} input sets cycled",
            "rows": N, "kv_lora_rank": D, "block_size": B, "input_sets_cycled": sets,
        },
        "kernel_us": {"dsa_latent_write_kernel": kern_ms * 1e3},
        "kernel_us_source": "HIP events around the timed region on the launch stream, / steps",
        # back-to-back 128-row launches: bound by the host's launch rate, so
        # this is an upper bound on the kernel's own duration at that size
        "region_us_per_launch_128_rows": small_ms * 1e3 / K,
        "arithmetic": "fp32 RMSNorm and scaling, hardware FP8 E4M3 conversion "
                      "(nearest, ties to even) after saturating to +-448",
        "roofline": {
            "bound": "hbm",
            "kernel": "dsa_latent_write_kernel",
            "achieved": gbps,
            "peak": HBM_PEAK_GBPS,
            "unit": "GB/s",
            "frac": gbps / HBM_PEAK_GBPS,
            "traffic": None,
            "algorithmic_bytes_per_launch": alg,
        },
    }
    measured = measured_traffic("bulk", "dsa_latent_write_kernel", "latent_write.hip")
    if measured is not None and N == 65536:
        result["roofline"]["traffic"] = measured
        result["roofline"]["traffic_unit"] = ("bytes per launch, rocprofv3 FETCH_SIZE + WRITE_SIZE "
                                              "scaled by a 256 MiB copy's readings")
    if args.cpu_rows > 0:
        result["cpu_baseline"] = cpu_baseline_writer(batches[0], weight, B, eps, kv_scale,
                                                     16 * args.cpu_rows)
    print(json.dumps(result), flush=True)


def cpu_baseline_writer(batch, weight, block_size, eps, kv_scale, nrows):
    """The CPU oracle's cache writer, as it stands (one thread), on the first
    `nrows` rows of the first input set."""
    import numpy as np
    import torch

    import oracle

    kv, sl = batch
    n = min(nrows, kv.shape[0])
    kv_bits = kv[:n].view(torch.int16).cpu().numpy().view(np.uint16)
    w_bits = weight.view(torch.int16).cpu().numpy().view(np.uint16)
    D = kv_bits.shape[1]
    # the sample's rows go to slots 0..n-1 of a compact host pool
    slots = np.arange(n, dtype=np.int64)
    pool = np.zeros(((n + block_size - 1) // block_size) * block_size * D, dtype=np.uint8)
    t = time.perf_counter()
    oracle.latent_write(kv_bits, w_bits, slots, pool, block_size=block_size,
                        cache_stride_bytes=0, eps=eps, inv_kv_scale=1.0 / kv_scale)
    dt = time.perf_counter() - t
    return {"value": n / dt, "unit": "rows/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} of {kv.shape[0]} rows of the first input set, float64 C "
                      f"oracle, {dt:.2f} s wall"}


if __name__ == "__main__":
    main()
