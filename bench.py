#!/usr/bin/env python3
"""Benchmark of the paged-KV decode step on one MI355X.

Workload: the Llama-70B-shaped layer (64 query / 8 KV heads, head_dim 128,
bf16, 16-token blocks, 32 sequences with context U[512, 4096], physical
blocks shuffled over a pool 1.2x the need).  One step = the slot-mapped append
of each sequence's current token (pkv_append) + paged decode attention over
its whole context (pkv_decode).  Inputs are resident in HBM before timing.
To keep the 256 MB Infinity Cache from serving repeated reads of the ~300 MB
of K/V, R copies of the paged state (each with its own block placement) are
rotated so that R * pool exceeds 1 GB.

Prints one JSON line (rank 0, N = 1).
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

METRIC = "paged decode effective KV GB/s (% of HBM peak) + seq-steps/s, 64q/8kv hd128"
HBM_PEAK_GBS = 8000.0


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def build_copies(batch, copies: int):
    """R independent paged states of the same logical batch."""
    from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows
    import paged_kv_cache_indirected_amd as pkv
    sh = batch.shape
    st = batch.seq_start()
    ids = list(range(batch.B))
    rows_k = np.concatenate([batch.k[st[b]:st[b + 1] - 1] for b in ids])
    rows_v = np.concatenate([batch.v[st[b]:st[b + 1] - 1] for b in ids])
    last = st[1:] - 1
    states = []
    for r in range(copies):
        cache = PagedCache(batch.pool_blocks, sh.Hkv, sh.block_size, sh.D, pkv.BF16,
                           pool_seed=batch.pool_seed + 7919 * r)
        cache.add_sequences(ids, batch.lens - 1, rows_k, rows_v)
        slots = cache.seqs.append_batch(ids)            # the step's bookkeeping (host)
        tables, lens, max_len = cache.tables(ids)
        import torch
        states.append(dict(
            cache=cache, tables=tables, lens=lens, max_len=max_len,
            slots=torch.from_numpy(slots).to("cuda"),
            k_new=to_device_rows(batch.k[last], pkv.BF16, "cuda"),
            v_new=to_device_rows(batch.v[last], pkv.BF16, "cuda"),
        ))
    return states


def cpu_baseline(batch, min_seconds: float = 10.0, max_reps: int = 400):
    """The fp64 oracle on the same workload, all host cores, timed around the
    compute only.  The sample is the whole decode step, repeated until at
    least min_seconds have elapsed (bounded by max_reps)."""
    import oracle
    threads = len(os.sched_getaffinity(0))
    oracle.decode(batch.q[:1], batch.k[:int(batch.lens[0])], batch.v[:int(batch.lens[0])],
                  batch.lens[:1], batch.shape.scale, threads=threads)  # load / warm
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(batch.q, batch.k, batch.v, batch.lens, batch.shape.scale, threads=threads)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds or reps >= max_reps:
            break
    sh = batch.shape
    step_bytes = float(batch.lens.sum()) * sh.Hkv * sh.D * 2 * sh.elem
    try:
        model = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if "model name" in l][0]
    except Exception:
        model = "unknown"
    return {"value": step_bytes * reps / el / 1e9, "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole decode step (B={batch.B}, all {batch.B * sh.Hq} (seq, head) rows) "
                      f"x {reps} repetitions, {el:.1f} s, fp64, cpu: {model}",
            "seq_steps_per_s": batch.B * reps / el}


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--splits", type=int, default=0, help="workgroups per KV head (0: library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    args = ap.parse_args()
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported "
              "(the paged-KV path here is single-GPU by design)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_indirected_amd as pkv
    import synth

    torch.cuda.set_device(0)
    batch = synth.cfg2()
    sh = batch.shape
    log(f"[bench] building {args.copies} paged copies of cfg2 (B={batch.B}, "
        f"sum L={int(batch.lens.sum())}, pool={batch.pool_blocks} blocks)")
    states = build_copies(batch, args.copies)
    from paged_kv_cache_indirected_amd.paged import to_device_rows
    q = to_device_rows(batch.q, pkv.BF16, "cuda")
    out = torch.empty((batch.B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    desc = states[0]["cache"].desc
    max_len = max(s["max_len"] for s in states)
    nbytes = pkv.decode_workspace_bytes(batch.B, sh.Hq, max_len, desc, args.splits)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    splits = args.splits or pkv.decode_num_splits(batch.B, sh.Hq, max_len, desc)

    def step(i):
        s = states[i % len(states)]
        c = s["cache"]
        pkv.append(s["k_new"], s["v_new"], s["slots"], c.k_cache, c.v_cache, c.desc)
        pkv.decode(q, c.k_cache, c.v_cache, s["tables"], s["lens"], sh.scale, out, c.desc,
                   max_len, workspace=ws, num_splits=args.splits)

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    t0 = torch.cuda.Event(enable_timing=True)
    t1 = torch.cuda.Event(enable_timing=True)
    t0.record()
    for i in range(args.steps):
        step(i)
    t1.record()
    torch.cuda.synchronize()
    ms_step = t0.elapsed_time(t1) / args.steps

    # Decode launches alone, each bracketed by events on the launch stream.
    n_dec = args.steps
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
           for _ in range(n_dec)]
    for i in range(n_dec):
        s = states[i % len(states)]
        c = s["cache"]
        evs[i][0].record()
        pkv.decode(q, c.k_cache, c.v_cache, s["tables"], s["lens"], sh.scale, out, c.desc,
                   max_len, workspace=ws, num_splits=args.splits)
        evs[i][1].record()
    torch.cuda.synchronize()
    dec_ms = np.array([a.elapsed_time(b) for a, b in evs])
    dec_avg = float(dec_ms.mean())

    kv_bytes = float(batch.lens.sum()) * sh.Hkv * sh.D * 2 * sh.elem
    gbs_step = kv_bytes / (ms_step * 1e-3) / 1e9
    gbs_dec = kv_bytes / (dec_avg * 1e-3) / 1e9
    res = {
        "metric": METRIC,
        "value": round(gbs_step, 1),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {
            "workload": "llama70b-shaped paged decode step: append 1 token + decode, B=32, "
                        "64q/8kv, d128, bf16, block 16, context U[512,4096], shuffled pool 1.2x",
            "global_batch": batch.B,
            "context_tokens": int(batch.lens.sum()),
            "pool_copies_rotated": len(states),
            "splits_per_kv_head": splits,
        },
        "pct_of_hbm_peak": round(100.0 * gbs_step / HBM_PEAK_GBS, 2),
        "seq_steps_per_s": round(batch.B / (ms_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "pkv_decode (balanced split pass + LSE merge)",
            "achieved": round(gbs_dec, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs_dec / HBM_PEAK_GBS, 4),
            "traffic": None,
            "algorithmic_bytes_per_launch": int(kv_bytes),
            "avg_launch_ms": round(dec_avg, 5),
            "p10_ms": round(float(np.percentile(dec_ms, 10)), 5),
            "p90_ms": round(float(np.percentile(dec_ms, 90)), 5),
        },
    }
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(batch)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
