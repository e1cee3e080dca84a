#!/usr/bin/env python3
"""Benchmark of the paged-KV attention path on one MI355X.

Headline workload: the Llama-70B-shaped layer (64 query / 8 KV heads,
head_dim 128, bf16, 16-token blocks, 32 sequences with context U[512, 4096],
physical blocks shuffled over a pool 1.2x the need).  One step = the
slot-mapped append of each sequence's current token (pkv_append) + paged
decode attention over its whole context (pkv_decode).  Inputs are resident in
HBM before timing.  To keep the 256 MB Infinity Cache from serving repeated
reads of the ~300 MB of K/V, R copies of the paged state (each with its own
block placement) are rotated so that R * pool exceeds 1 GB.

The other workloads are measured in the same run and reported under
"workloads": the continuous-batching step (256 sequences, 32-token blocks,
churn between steps), prefix-sharing decode (128 sequences on one 2048-token
shared prefix), chunked prefill on MFMA mixed with decode, plus the
bandwidth probes that bound the gather (contiguous read, paged tile read).

Prints one JSON line (N = 1).
"""
from __future__ import annotations

import argparse
import ctypes
import hashlib
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "paged decode effective KV GB/s (% of HBM peak) + seq-steps/s, 64q/8kv hd128"
HBM_PEAK_GBS = 8000.0
MFMA_BF16_PEAK_TFLOPS = 2500.0
PMC_FILE = os.path.join(ROOT, "profiles", "decode_cfg2_pmc_traffic.json")
PMC_INDIRECTION_FILE = os.path.join(ROOT, "profiles", "decode_cfg2_indirection_pmc.json")
PMC_CFG4_FILE = os.path.join(ROOT, "profiles", "decode_cfg4_pmc_traffic.json")
DECODE_SRC = os.path.join(ROOT, "paged_kv_cache_indirected_amd", "csrc", "decode.hip")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kv_row_bytes(sh):
    return sh.Hkv * sh.D * 2 * sh.elem


class Timer:
    """HIP events on the current (launch) stream around n calls of fn."""

    def __init__(self):
        import torch
        self.torch = torch

    def per_call(self, fn, n, warmup=3):
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(n)]
        for i in range(n):
            evs[i][0].record()
            fn()
            evs[i][1].record()
        torch.cuda.synchronize()
        return np.array([a.elapsed_time(b) for a, b in evs]) * 1e-3   # seconds

    def amortized(self, fn, n, warmup=3):
        """Seconds per call over n back-to-back calls bracketed by one pair
        of events (the launch overhead of each call overlaps the previous
        call's execution, as in a serving loop)."""
        torch = self.torch
        for _ in range(warmup):
            fn()
        torch.cuda.synchronize()
        a = torch.cuda.Event(enable_timing=True)
        b = torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(n):
            fn()
        b.record()
        torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e-3 / n


def decode_side_bytes(lens, sh, splits, out_bytes=4):
    """Bytes a pkv_decode call moves besides the K/V rows (the algorithmic
    bytes): q rows, the output, block-table entries and context lengths, and
    the split pieces' partial states (written by the split pass, read by the
    merge).  The pieces follow the split pass's cut: a cost line of
    blocks + piece_cost per sequence boundary cut into `splits` equal ranges
    per KV head; a sequence whose blocks span several ranges leaves one
    partial (G x (D + 2) floats) per range and KV head."""
    bs, D, Hq, Hkv = sh.block_size, sh.D, sh.Hq, sh.Hkv
    esz = 4 if sh.dtype == "f32" else 2
    G = Hq // Hkv
    L = np.asarray(lens, dtype=np.int64)
    nb = (L + bs - 1) // bs
    pref = np.concatenate([[0], np.cumsum(nb)])
    B, T = len(L), int(pref[-1])
    pc = max(1, 147456 // (2 * bs * D * esz))
    Ct = T + pc * B

    def owner(c):
        return ((c + 1) * splits + Ct - 1) // Ct - 1
    pieces = 0
    for b in range(B):
        sb, se = int(pref[b]), int(pref[b + 1])
        if se > sb:
            wf, wl = owner(sb + pc * b), owner(se - 1 + pc * b)
            pieces += (wl - wf + 1) if wl > wf else 0
    part = pieces * Hkv * G * (D + 2) * 4
    side = {"q": B * Hq * D * esz, "out": B * Hq * D * out_bytes,
            "block_tables": T * 4 * Hkv, "context_lens_and_prefix_sums": B * 4 + 2 * (B + 1) * 4,
            "partials_written": part, "partials_read": part}
    side["total"] = int(sum(side.values()))
    side["split_pieces_per_kv_head"] = pieces
    side["note"] = ("block-table entries counted once per KV head (each head's workgroups read "
                    "their ranges' ids); partial states of sequences cut between workgroups")
    return side


def paged_state(batch, pool_seed, device="cuda"):
    """One paged copy of a decode batch: every row but each sequence's last
    loaded through the pool and pkv_append; the step's last token is left for
    the timed append.  Returns a dict of device tensors."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows
    sh = batch.shape
    st = batch.seq_start()
    ids = list(range(batch.B))
    dt = pkv.F32 if sh.dtype == "f32" else pkv.BF16
    cache = PagedCache(batch.pool_blocks, sh.Hkv, sh.block_size, sh.D, dt, pool_seed=pool_seed)
    rows_k = np.concatenate([batch.k[st[b]:st[b + 1] - 1] for b in ids])
    rows_v = np.concatenate([batch.v[st[b]:st[b + 1] - 1] for b in ids])
    cache.add_sequences(ids, batch.lens - 1, rows_k, rows_v)
    slots = cache.seqs.append_batch(ids)            # the step's bookkeeping (host)
    tables, lens, max_len = cache.tables(ids)
    last = st[1:] - 1
    return dict(cache=cache, tables=tables, lens=lens, max_len=max_len,
                slots=torch.from_numpy(slots).to(device),
                k_new=to_device_rows(batch.k[last], dt, device),
                v_new=to_device_rows(batch.v[last], dt, device),
                q=to_device_rows(batch.q, dt, device))


def workspace(B, Hq, max_len, desc, splits):
    import torch
    import paged_kv_cache_indirected_amd as pkv
    n = pkv.decode_workspace_bytes(B, Hq, max_len, desc, splits)
    return torch.empty(max(n, 1), dtype=torch.uint8, device="cuda")


class PrefillWorkspace:
    """The workspace pkv_prefill_chunk asks for (key-split states), grown on
    demand; a larger buffer than a call needs is fine."""

    def __init__(self):
        self.buf = None

    def get(self, S, Hq, max_query_len, desc):
        import torch
        import paged_kv_cache_indirected_amd as pkv
        n = pkv.prefill_workspace_bytes(S, Hq, max_query_len, desc)
        if n and (self.buf is None or self.buf.numel() < n):
            self.buf = torch.empty(n, dtype=torch.uint8, device="cuda")
        return self.buf if n else None


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
    step_bytes = float(batch.lens.sum()) * kv_row_bytes(batch.shape)
    try:
        model = [l.split(":", 1)[1].strip() for l in open("/proc/cpuinfo") if "model name" in l][0]
    except Exception:
        model = "unknown"
    return {"value": round(step_bytes * reps / el / 1e9, 3), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"whole decode step of the Llama-70B-shaped batch (B={batch.B}, all "
                      f"{batch.B * batch.shape.Hq} (seq, head) rows, {int(batch.lens.sum())} "
                      f"context tokens) x {reps} repetitions in {el:.1f} s, fp64, cpu: {model}",
            "seq_steps_per_s": round(batch.B * reps / el, 2)}


def _pmc_record(path):
    """A committed PMC summary, if it was taken on the current decode source
    (its decode.hip SHA-256 matches); else None."""
    try:
        rec = json.load(open(path))
    except (OSError, ValueError):
        return None
    sha = hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest()
    return rec if rec.get("decode_hip_sha256") == sha else None


def pmc_traffic(launch_bytes):
    """HBM bytes per decode call from the committed PMC summary, if it was
    taken on the current decode source; else None."""
    rec = _pmc_record(PMC_FILE)
    return None if rec is None else rec.get("hbm_bytes_per_call")


# ---------------------------------------------------------------------------
# Workloads beyond the headline (reported under "workloads").

def bench_probes(timer):
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_indirected_amd", "libpkv_probe.so"))
    P = ctypes.c_void_p
    lib.pkv_probe_stream_read.argtypes = [P, ctypes.c_size_t, P, ctypes.c_int, P]
    lib.pkv_probe_tile_read.argtypes = [P, P, P, ctypes.c_int64, ctypes.c_int, P, ctypes.c_int, P]
    st = torch.cuda.current_stream().cuda_stream
    sink = torch.zeros(1 << 16, dtype=torch.int32, device="cuda")
    n = 2 << 30
    buf = torch.zeros(n // 2, dtype=torch.int16, device="cuda")
    t = timer.per_call(lambda: lib.pkv_probe_stream_read(buf.data_ptr(), n // 16,
                                                         sink.data_ptr(), 2048, st), 20)
    del buf
    return {"stream_read_GBps": round(n / float(np.median(t)) / 1e9, 1),
            "note": "contiguous read of 2 GiB, 2048 workgroups"}, lib, sink


def bench_tile_probe(lib, sink, states, sh, kv_bytes, timer, grid=256):
    """The decode's access shape without arithmetic: whole (block, head)
    tiles of K and V of the same shuffled pools, in sequence order."""
    import torch
    st = torch.cuda.current_stream().cuda_stream
    lists = []
    for s in states:
        tab = s["tables"].cpu().numpy()
        lens = s["lens"].cpu().numpy()
        ids = []
        for b in range(len(lens)):
            nb = (int(lens[b]) + sh.block_size - 1) // sh.block_size
            for blk in tab[b, :nb]:
                ids.extend(int(blk) * sh.Hkv + g for g in range(sh.Hkv))
        lists.append(torch.tensor(ids, dtype=torch.int64, device="cuda"))
    tile = sh.block_size * sh.D * sh.elem
    i = [0]

    def run():
        s = states[i[0] % len(states)]
        t = lists[i[0] % len(states)]
        i[0] += 1
        lib.pkv_probe_tile_read(s["cache"].k_cache.data_ptr(), s["cache"].v_cache.data_ptr(),
                                t.data_ptr(), t.numel(), tile, sink.data_ptr(), grid, st)
    t = timer.per_call(run, 40)
    return round(kv_bytes / float(np.median(t)) / 1e9, 1)


def identity_states(batch, copies):
    """Paged copies of a decode batch whose sequences' rows are appended
    whole, in order, from an ascending free list: each sequence's blocks are
    consecutive and ascending (the placement a contiguous per-sequence cache
    would have)."""
    import paged_kv_cache_indirected_amd as pkv
    from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows
    sh = batch.shape
    out = []
    for _ in range(copies):
        c = PagedCache(batch.pool_blocks, sh.Hkv, sh.block_size, sh.D, pkv.BF16, pool_seed=0)
        ids = list(range(batch.B))
        c.add_sequences(ids, batch.lens, batch.k, batch.v)
        tables, lens, mx = c.tables(ids)
        tab = tables.cpu().numpy()
        for b in range(batch.B):
            nb = (int(batch.lens[b]) + sh.block_size - 1) // sh.block_size
            assert np.all(np.diff(tab[b, :nb]) == 1), "identity placement is not contiguous"
        out.append(dict(cache=c, tables=tables, lens=lens, max_len=mx,
                        q=to_device_rows(batch.q, pkv.BF16, "cuda")))
    return out


def bench_indirection(timer, batch, shuffled, splits, calls=200):
    """The cost of the logical-to-physical block map: the Llama-70B-shaped
    decode call over the same rows placed in shuffled blocks (the
    headline's copies) and in an identity placement (every sequence's
    blocks consecutive and ascending: what a contiguous per-sequence cache
    would read), the same number of copies rotated for each.  HBM bytes per
    call by counter come from the committed summary when it matches the
    decode source."""
    import paged_kv_cache_indirected_amd as pkv
    sh = batch.shape
    identity = identity_states(batch, len(shuffled))
    max_len = max(s["max_len"] for s in shuffled + identity)
    desc = shuffled[0]["cache"].desc
    ws = workspace(batch.B, sh.Hq, max_len, desc, splits)
    import torch
    res_out = torch.empty((batch.B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    kv = float(batch.lens.sum()) * kv_row_bytes(sh)

    def timed(states):
        it = [0]

        def call():
            st = states[it[0] % len(states)]
            it[0] += 1
            c = st["cache"]
            pkv.decode(st["q"], c.k_cache, c.v_cache, st["tables"], st["lens"], sh.scale,
                       res_out, c.desc, max_len, workspace=ws, num_splits=splits)
        return timer.per_call(call, calls, warmup=10)
    ts, ti = [], []
    for _ in range(2):                       # alternate: drift hits both alike
        ts.append(timed(shuffled))
        ti.append(timed(identity))
    t_s = float(np.median(np.concatenate(ts)))
    t_i = float(np.median(np.concatenate(ti)))
    r = {"workload": "the Llama-70B-shaped decode call (B=32, 64q/8kv, d128, bf16, block 16) "
                     "over shuffled blocks vs an identity placement (each sequence's blocks "
                     f"consecutive), {len(shuffled)} copies of each rotated",
         "shuffled_ms": round(1e3 * t_s, 5), "identity_ms": round(1e3 * t_i, 5),
         "shuffled_GBps": round(kv / t_s / 1e9, 1), "identity_GBps": round(kv / t_i / 1e9, 1),
         "shuffled_over_identity_time": round(t_s / t_i, 4)}
    rec = _pmc_record(PMC_INDIRECTION_FILE)
    if rec is not None:
        r["hbm_fetch_bytes_per_call"] = {"shuffled": rec["shuffled_fetch_bytes_per_call"],
                                         "identity": rec["identity_fetch_bytes_per_call"]}
    del identity
    return r


def bench_metadata(timer, batch, steps=50):
    """Per-step metadata of the Llama-70B-shaped step (a2): the host
    bookkeeping (one new token per sequence, then block tables and lengths)
    written into pinned memory, and its one asynchronous copy to the device,
    each timed alone (the GPU idle), beside the decode step's kernel time."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    from paged_kv_cache_indirected_amd.paged import StepMetadata
    sh = batch.shape
    st = paged_state(batch, batch.pool_seed)
    cache = st["cache"]
    ids = list(range(batch.B))
    stride = int(st["tables"].shape[1]) + (steps + sh.block_size) // sh.block_size + 1
    md = StepMetadata(batch.B, stride, depth=4)
    host_s, h2d_s = [], []
    ids = np.arange(batch.B, dtype=np.int64)
    ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for i in range(steps + 5):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        h = md.fill(cache.seqs, ids)
        t1 = time.perf_counter()
        md.upload(h, timing=ev)
        torch.cuda.synchronize()
        if i >= 5:
            host_s.append(t1 - t0)
            h2d_s.append(ev[0].elapsed_time(ev[1]) * 1e-3)
    nbytes = 4 * batch.B * (stride + 2)
    del st
    return {"workload": f"decode-step metadata of B={batch.B} sequences: slots, context lengths "
                        f"and block tables ({stride} entries per row), pinned host -> device",
            "bytes_per_step": nbytes,
            "host_bookkeeping_us": round(1e6 * float(np.median(host_s)), 2),
            "h2d_us": round(1e6 * float(np.median(h2d_s)), 2),
            "note": "outside the kernels' timed region; a serving loop overlaps the copy with "
                    "the previous step's kernels (non-blocking, stream-ordered)"}


def cpu_single_thread(batch, min_seconds: float = 3.0):
    """The oracle on one host thread, whole decode step, repeated until
    min_seconds have elapsed (at least once)."""
    import oracle
    reps, t0 = 0, time.perf_counter()
    while True:
        oracle.decode(batch.q, batch.k, batch.v, batch.lens, batch.shape.scale, threads=1)
        reps += 1
        el = time.perf_counter() - t0
        if el >= min_seconds:
            break
    step_bytes = float(batch.lens.sum()) * kv_row_bytes(batch.shape)
    return {"value": round(step_bytes * reps / el / 1e9, 4), "unit": "GB/s", "cores": 1,
            "seq_steps_per_s": round(batch.B * reps / el, 2),
            "sample": f"{batch.name}: whole decode step (B={batch.B}, "
                      f"{int(batch.lens.sum())} context tokens) x {reps} in {el:.1f} s"}


def bench_cfg3(timer, steps, splits):
    """Continuous-batching steps: 256 sequences, 32-token blocks; each step
    appends one token per sequence and decodes; between steps 10% of the
    sequences finish and are replaced (host bookkeeping + untimed fill)."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    import synth
    from paged_kv_cache_indirected_amd.paged import PagedCache, StepMetadata, to_device_rows
    b0 = synth.cfg3_initial()
    sh = b0.shape
    st = b0.seq_start()
    cache = PagedCache(b0.pool_blocks, sh.Hkv, sh.block_size, sh.D, pkv.BF16,
                       pool_seed=b0.pool_seed)
    ids = list(range(b0.B))
    rows_k = np.concatenate([b0.k[st[b]:st[b + 1] - 1] for b in ids])
    rows_v = np.concatenate([b0.v[st[b]:st[b + 1] - 1] for b in ids])
    cache.add_sequences(ids, b0.lens - 1, rows_k, rows_v)
    del rows_k, rows_v
    next_id = b0.B
    stride = (8192 + 1 + steps + sh.block_size) // sh.block_size + 1
    out = torch.empty((b0.B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    ws = workspace(b0.B, sh.Hq, stride * sh.block_size, cache.desc, splits)
    times, times_fused, times_b2b, kvb = [], [], [], 0.0
    md = StepMetadata(b0.B, stride, depth=4)
    md_host, md_h2d = [], []
    md_ev = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
    for step in range(1, steps + 1):
        kn, vn, qn = synth.cfg3_step_rows(step, b0.B, sh)
        kn, vn, qn = (to_device_rows(x, pkv.BF16, "cuda") for x in (kn, vn, qn))
        # The step's metadata: bookkeeping into pinned memory, one async copy
        # (each timed alone here; a serving loop overlaps the copy with the
        # previous step's kernels).
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        h = md.fill(cache.seqs, ids)
        md_host.append(time.perf_counter() - t0)
        tab, lens, slots, mx = md.upload(h, timing=md_ev)
        torch.cuda.synchronize()
        md_h2d.append(md_ev[0].elapsed_time(md_ev[1]) * 1e-3)

        def run():
            pkv.append(kn, vn, slots, cache.k_cache, cache.v_cache, cache.desc)
            pkv.decode(qn, cache.k_cache, cache.v_cache, tab, lens, sh.scale, out, cache.desc, mx,
                       workspace=ws, num_splits=splits)

        def run_fused():
            pkv.append_decode(kn, vn, slots, qn, cache.k_cache, cache.v_cache, tab, lens,
                              sh.scale, out, cache.desc, mx, workspace=ws, num_splits=splits)
        # The step's append writes the same bytes every time, so both forms
        # can be timed on the same state.
        times.append(float(np.median(timer.per_call(run, 5, warmup=1))))
        times_fused.append(float(np.median(timer.per_call(run_fused, 5, warmup=1))))
        # The same fused step enqueued back to back, as a serving loop runs
        # ahead of the GPU (each call above also waits for its own launch).
        times_b2b.append(timer.amortized(run_fused, 10, warmup=1))
        kvb += float(lens.sum().item()) * kv_row_bytes(sh)
        ev = synth.cfg3_churn(step, b0.B, sh)
        for i, pos in enumerate(ev.finished):
            cache.release(ids[pos])
            ids[pos] = next_id
            cache.add_sequences([next_id], [int(ev.new_lens[i])], ev.new_k[i], ev.new_v[i])
            next_id += 1
    # The same bookkeeping back to back (8 more appended tokens per sequence,
    # no churn or kernels in between): the figures above include whatever
    # the churn left cold in the host caches.
    warm_host, warm_h2d = [], []
    for _ in range(8):
        torch.cuda.synchronize()
        t0 = time.perf_counter()
        h = md.fill(cache.seqs, ids)
        warm_host.append(time.perf_counter() - t0)
        md.upload(h, timing=md_ev)
        torch.cuda.synchronize()
        warm_h2d.append(md_ev[0].elapsed_time(md_ev[1]) * 1e-3)
    t_sep, t_fused = float(np.sum(times)), float(np.sum(times_fused))
    t = min(t_sep, t_fused)
    return {"workload": "continuous-batching step: append 1 token + decode, B=256, 64q/8kv, "
                        "d128, bf16, block 32, log-normal context (median 1024), 10% churn/step",
            "step_calls": "pkv_append_decode" if t_fused <= t_sep else "pkv_append + pkv_decode",
            "ms_per_step_append_then_decode": round(1e3 * t_sep / steps, 4),
            "ms_per_step_fused_append_decode": round(1e3 * t_fused / steps, 4),
            "steps": steps, "ms_per_step": round(1e3 * t / steps, 4),
            "kv_GBps": round(kvb / t / 1e9, 1),
            "seq_steps_per_s": round(b0.B * steps / t, 1),
            "pct_of_hbm_peak": round(100 * kvb / t / 1e9 / HBM_PEAK_GBS, 2),
            "ms_per_step_back_to_back": round(1e3 * float(np.sum(times_b2b)) / steps, 4),
            "kv_GBps_back_to_back": round(kvb / float(np.sum(times_b2b)) / 1e9, 1),
            "pct_of_hbm_peak_back_to_back": round(
                100 * kvb / float(np.sum(times_b2b)) / 1e9 / HBM_PEAK_GBS, 2),
            "metadata": {"bytes_per_step": 4 * b0.B * (stride + 2),
                         "host_bookkeeping_us": round(1e6 * float(np.median(md_host)), 2),
                         "h2d_us": round(1e6 * float(np.median(md_h2d)), 2),
                         "host_bookkeeping_us_back_to_back": round(
                             1e6 * float(np.median(warm_host)), 2),
                         "h2d_us_back_to_back": round(1e6 * float(np.median(warm_h2d)), 2),
                         "note": "slots, context lengths and block tables written by the host "
                                 "bookkeeping into pinned memory and copied asynchronously; "
                                 "outside the step's timed kernels.  First pair: each step "
                                 "between churn and kernels (median of the steps); second: "
                                 "8 more steps' bookkeeping back to back"}}


def bench_decode_sweep(timer):
    """Decode at batch sizes 1 .. 128, every sequence at context 4096
    (64q/8kv, d128, bf16, 16-token blocks): the automatic split (about one
    workgroup per CU, sequences cut across workgroups and merged) against
    one workgroup per (sequence, KV head) (num_splits = B: with equal
    lengths every range is exactly one sequence, nothing is merged).  Each
    point rotates enough shuffled copies that they exceed the 256 MB
    Infinity Cache.  The rows of one 4096-token sequence are reused for every
    sequence (the values do not change the work)."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    import synth
    L, Bmax = 4096, 128
    base = synth.cfg2(B=1)
    sh = base.shape
    g = synth.rng(2, synth.S_K, 9)
    rk = synth.normal(g, (L, sh.Hkv, sh.D), sh.dtype)
    rv = synth.normal(synth.rng(2, synth.S_V, 9), (L, sh.Hkv, sh.D), sh.dtype)
    res = {}
    for B in (1, 2, 4, 8, 16, 32, 64, 128):
        lens = np.full(B, L, dtype=np.int64)
        b = synth.DecodeBatch(2, "sweep", sh, lens, synth.normal(synth.rng(2, synth.S_Q, 9, B),
                              (B, sh.Hq, sh.D), sh.dtype), np.tile(rk, (B, 1, 1)),
                              np.tile(rv, (B, 1, 1)), pool_blocks=B * (L // sh.block_size) + 8,
                              pool_seed=base.pool_seed)
        kv = float(B * L) * kv_row_bytes(sh)
        R = int(min(64, max(1, np.ceil(1.1e9 / kv))))
        states = [paged_state(b, b.pool_seed + 7919 * r) for r in range(R)]
        for st in states:
            c = st["cache"]
            pkv.append(st["k_new"], st["v_new"], st["slots"], c.k_cache, c.v_cache, c.desc)
        out = torch.empty((B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
        desc = states[0]["cache"].desc
        entry = {"copies": R}
        for label, W in (("auto_split", 0), ("one_wg_per_seq", B)):
            ws = workspace(B, sh.Hq, L, desc, W)
            it = [0]

            def call():
                st = states[it[0] % R]
                it[0] += 1
                c = st["cache"]
                pkv.decode(st["q"], c.k_cache, c.v_cache, st["tables"], st["lens"], sh.scale, out,
                           desc, L, workspace=ws, num_splits=W)
            t = float(np.median(timer.per_call(call, max(2 * R, 40), warmup=R)))
            ta = timer.amortized(call, max(4 * R, 200), warmup=R)
            entry[label] = {"ms": round(1e3 * t, 4), "kv_GBps": round(kv / t / 1e9, 1),
                            "pct_of_hbm_peak": round(100 * kv / t / 1e9 / HBM_PEAK_GBS, 2),
                            "ms_back_to_back": round(1e3 * ta, 4),
                            "pct_of_hbm_peak_back_to_back":
                                round(100 * kv / ta / 1e9 / HBM_PEAK_GBS, 2)}
        entry["split_speedup"] = round(entry["one_wg_per_seq"]["ms"] / entry["auto_split"]["ms"], 3)
        res[f"B{B}"] = entry
        del states
        torch.cuda.empty_cache()
    res["workload"] = ("decode at B = 1..128, every context 4096, 64q/8kv, d128, bf16, block 16: "
                       "automatic split vs one workgroup per (sequence, KV head)")
    res["timing"] = ("ms: median of single calls, each bracketed by its own events; "
                     "ms_back_to_back: events around a run of back-to-back calls over the "
                     "rotated copies, per call")
    return res


def bench_cfg4(timer, splits):
    """Prefix-sharing decode: 128 sequences share one 2048-token prefix's
    physical blocks; logical bytes count the prefix once per sequence."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    import synth
    from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows
    b = synth.cfg4()
    sh = b.shape
    st = b.seq_start()
    P = b.prefix_len
    cache = PagedCache(b.pool_blocks, sh.Hkv, sh.block_size, sh.D, pkv.BF16,
                       pool_seed=b.pool_seed)
    cache.add_sequences([-1], [P], b.k[:P], b.v[:P])
    for s in range(b.B):
        cache.add_shared(s, -1, P)
        cache.extend(s, b.k[st[s] + P:st[s + 1]], b.v[st[s] + P:st[s + 1]])
    tab, lens, mx = cache.tables(list(range(b.B)))
    q = to_device_rows(b.q, pkv.BF16, "cuda")
    out = torch.empty((b.B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    ws = workspace(b.B, sh.Hq, mx, cache.desc, splits)
    t = float(np.median(timer.per_call(
        lambda: pkv.decode(q, cache.k_cache, cache.v_cache, tab, lens, sh.scale, out, cache.desc,
                           mx, workspace=ws, num_splits=splits), 30)))
    logical = float(b.lens.sum()) * kv_row_bytes(sh)
    unique = float(P + (b.lens - P).sum()) * kv_row_bytes(sh)
    # The same step through the cascade decode: the shared prefix's blocks
    # once for all sequences (non-causal MFMA pass), then the own blocks.
    nbp = P // sh.block_size
    pblocks = torch.tensor(cache.seqs.block_ids(-1)[:nbp], dtype=torch.int32, device="cuda")
    tab_s = tab[:, nbp:].contiguous()
    lens_s = (lens - P).to(torch.int32).contiguous()
    mx_s = int(lens_s.max().item())
    cws = torch.empty(pkv.decode_cascade_workspace_bytes(b.B, sh.Hq, P, mx_s, cache.desc),
                      dtype=torch.uint8, device="cuda")
    def cascade():
        pkv.decode_cascade(q, cache.k_cache, cache.v_cache, pblocks, P, tab_s, lens_s,
                           sh.scale, out, cache.desc, mx_s, workspace=cws)
    tc = float(np.median(timer.per_call(cascade, 30)))
    # Back to back, as a serving loop enqueues ahead of the GPU: the host
    # launch path of each call then overlaps the previous call's kernels.
    t_b2b = timer.amortized(
        lambda: pkv.decode(q, cache.k_cache, cache.v_cache, tab, lens, sh.scale, out, cache.desc,
                           mx, workspace=ws, num_splits=splits), 30)
    tc_b2b = timer.amortized(cascade, 30)
    return {"workload": "prefix-sharing decode: B=128 on one shared 2048-token prefix + "
                        "U[64,512] private, 64q/8kv, d128, bf16, block 16",
            "ms_per_call": round(1e3 * t, 4),
            "logical_kv_GBps": round(logical / t / 1e9, 1),
            "unique_kv_GBps": round(unique / t / 1e9, 1),
            "seq_steps_per_s": round(b.B / t, 1),
            "cascade_ms_per_call": round(1e3 * tc, 4),
            "cascade_unique_kv_GBps": round(unique / tc / 1e9, 1),
            "cascade_speedup": round(t / tc, 3),
            "ms_per_call_back_to_back": round(1e3 * t_b2b, 4),
            "cascade_ms_per_call_back_to_back": round(1e3 * tc_b2b, 4),
            "cascade_speedup_back_to_back": round(t_b2b / tc_b2b, 3),
            "logical_kv_bytes": logical, "unique_kv_bytes": unique,
            "hbm_bytes_by_counter": (lambda r: None if r is None else {
                "plain": r["plain_hbm_bytes_per_call"],
                "cascade": r["cascade_hbm_bytes_per_call"]})(_pmc_record(PMC_CFG4_FILE)),
            "note": "logical bytes read the shared prefix once per sequence; repeated prefix "
                    "tiles are served from L2/Infinity Cache, so logical GB/s can exceed HBM"}


def bench_cfg5(timer, splits):
    """Chunked prefill (4 x 512-token causal chunks on MFMA) in the same step
    as 64 decode sequences."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    import synth
    from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows
    pre, dec = synth.cfg5()
    sh = pre.shape
    pc = PagedCache(pre.pool_blocks, sh.Hkv, sh.block_size, sh.D, pkv.BF16,
                    pool_seed=pre.pool_seed)
    ids = list(range(len(pre.chunk)))
    lsum = pre.prior + pre.chunk
    qs0 = np.concatenate([[0], np.cumsum(lsum)])
    prior_k = np.concatenate([pre.k[qs0[s]:qs0[s] + pre.prior[s]] for s in ids])
    prior_v = np.concatenate([pre.v[qs0[s]:qs0[s] + pre.prior[s]] for s in ids])
    pc.add_sequences(ids, pre.prior, prior_k, prior_v)
    chunk_slots = np.concatenate([pc.seqs.append(s, int(pre.chunk[s])) for s in ids])
    ck = to_device_rows(np.concatenate([pre.k[qs0[s] + pre.prior[s]:qs0[s + 1]] for s in ids]),
                        pkv.BF16, "cuda")
    cv = to_device_rows(np.concatenate([pre.v[qs0[s] + pre.prior[s]:qs0[s + 1]] for s in ids]),
                        pkv.BF16, "cuda")
    cslots = torch.from_numpy(chunk_slots.astype(np.int32)).to("cuda")
    ptab, plens, pmx = pc.tables(ids)
    pq = to_device_rows(pre.q, pkv.BF16, "cuda")
    qsl = torch.from_numpy(pre.query_start.astype(np.int32)).to("cuda")
    pout = torch.empty(tuple(pq.shape), dtype=torch.float32, device="cuda")
    ds = paged_state(dec, dec.pool_seed)
    dout = torch.empty((dec.B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    dc = ds["cache"]
    ws = workspace(dec.B, sh.Hq, ds["max_len"], dc.desc, splits)
    C = int(pre.chunk.max())
    pws = PrefillWorkspace().get(len(pre.chunk), sh.Hq, C, pc.desc)

    def prefill():
        pkv.prefill_chunk(pq, qsl, pc.k_cache, pc.v_cache, ptab, plens, sh.scale, pout, pc.desc,
                          C, pmx, workspace=pws)

    def decode():
        pkv.decode(ds["q"], dc.k_cache, dc.v_cache, ds["tables"], ds["lens"], sh.scale, dout,
                   dc.desc, ds["max_len"], workspace=ws, num_splits=splits)

    def step():
        pkv.append(ck, cv, cslots, pc.k_cache, pc.v_cache, pc.desc)
        pkv.append(ds["k_new"], ds["v_new"], ds["slots"], dc.k_cache, dc.v_cache, dc.desc)
        prefill()
        decode()
    # The same step with the decode on a second stream (default priority):
    # the MFMA-bound prefill and the HBM-bound decode run side by side.
    side = torch.cuda.Stream()

    def step_two_streams():
        main = torch.cuda.current_stream()
        ev0 = torch.cuda.Event()
        ev0.record(main)
        side.wait_event(ev0)
        pkv.append(ck, cv, cslots, pc.k_cache, pc.v_cache, pc.desc)
        prefill()
        with torch.cuda.stream(side):
            pkv.append(ds["k_new"], ds["v_new"], ds["slots"], dc.k_cache, dc.v_cache, dc.desc,
                       stream=side)
            pkv.decode(ds["q"], dc.k_cache, dc.v_cache, ds["tables"], ds["lens"], sh.scale, dout,
                       dc.desc, ds["max_len"], workspace=ws, num_splits=splits, stream=side)
        ev1 = torch.cuda.Event()
        ev1.record(side)
        main.wait_event(ev1)
    def step_two_streams_decode_first():
        main = torch.cuda.current_stream()
        ev0 = torch.cuda.Event()
        ev0.record(main)
        side.wait_event(ev0)
        with torch.cuda.stream(side):
            pkv.append(ds["k_new"], ds["v_new"], ds["slots"], dc.k_cache, dc.v_cache, dc.desc,
                       stream=side)
            pkv.decode(ds["q"], dc.k_cache, dc.v_cache, ds["tables"], ds["lens"], sh.scale, dout,
                       dc.desc, ds["max_len"], workspace=ws, num_splits=splits, stream=side)
        pkv.append(ck, cv, cslots, pc.k_cache, pc.v_cache, pc.desc)
        prefill()
        ev1 = torch.cuda.Event()
        ev1.record(side)
        main.wait_event(ev1)
    t_pre = float(np.median(timer.per_call(prefill, 10)))
    t_dec = float(np.median(timer.per_call(decode, 20)))
    t_step = float(np.median(timer.per_call(step, 10)))
    t_step2 = float(np.median(timer.per_call(step_two_streams, 10)))
    t_step3 = float(np.median(timer.per_call(step_two_streams_decode_first, 10)))
    flops = sum(4.0 * sh.Hq * sh.D * (int(c) * int(p) + int(c) * (int(c) + 1) / 2)
                for p, c in zip(pre.prior, pre.chunk))
    dbytes = float(dec.lens.sum()) * kv_row_bytes(sh)
    return {"workload": "chunked prefill mixed with decode: 4 x 512-token causal chunks over "
                        "prior U[0,7680] (MFMA) + 64 decode seqs U[256,8192], 64q/8kv, d128, "
                        "bf16, block 16",
            "prior_tokens": [int(x) for x in pre.prior],
            "prefill_ms": round(1e3 * t_pre, 4),
            "prefill_TFLOPs": round(flops / t_pre / 1e12, 1),
            "prefill_mfma_frac": round(flops / t_pre / 1e12 / MFMA_BF16_PEAK_TFLOPS, 4),
            "prefill_algorithmic_GFLOP": round(flops / 1e9, 2),
            "decode_ms": round(1e3 * t_dec, 4),
            "decode_kv_GBps": round(dbytes / t_dec / 1e9, 1),
            "step_ms": round(1e3 * t_step, 4),
            "step_note": "append of 2048 chunk rows + 64 decode rows, prefill, decode; "
                         "one stream",
            "step_two_streams_ms": round(1e3 * t_step2, 4),
            "step_two_streams_note": "prefill (with its append) on the launch stream, decode "
                                     "(with its append) on a second stream, joined by events",
            "step_two_streams_decode_first_ms": round(1e3 * t_step3, 4),
            "short_chunk": bench_short_chunk(timer)}


def bench_short_chunk(timer):
    """One sequence prefilling a 64-token chunk over 8000 prior tokens
    (64q/8kv, d128, bf16, block 16): 32 workgroups, far fewer than the CUs.
    Timed as one pass per workgroup (no workspace) and with the keys split
    (the workspace pkv_prefill_chunk asks for)."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    import synth
    from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows
    b = synth.custom_prefill(9001, prior=[8000], chunk=[64], Hq=64, Hkv=8, D=128, block_size=16)
    sh = b.shape
    cache = PagedCache(b.pool_blocks, sh.Hkv, sh.block_size, sh.D, pkv.BF16,
                       pool_seed=b.pool_seed)
    cache.add_sequences([0], b.lens, b.k, b.v)
    tab, lens, mx = cache.tables([0])
    q = to_device_rows(b.q, pkv.BF16, "cuda")
    qs = torch.tensor([0, 64], dtype=torch.int32, device="cuda")
    out = torch.empty(tuple(q.shape), dtype=torch.float32, device="cuda")
    ws = PrefillWorkspace().get(1, sh.Hq, 64, cache.desc)

    def run(w):
        return lambda: pkv.prefill_chunk(q, qs, cache.k_cache, cache.v_cache, tab, lens,
                                         sh.scale, out, cache.desc, 64, mx, workspace=w)
    t1 = float(np.median(timer.per_call(run(None), 30)))
    t2 = float(np.median(timer.per_call(run(ws), 30)))
    flops = 4.0 * sh.Hq * sh.D * (64 * 8000 + 64 * 65 / 2)
    return {"workload": "one 64-token chunk over 8000 prior tokens, 64q/8kv, d128, bf16",
            "single_pass_ms": round(1e3 * t1, 4),
            "key_split_ms": round(1e3 * t2, 4),
            "key_split_TFLOPs": round(flops / t2 / 1e12, 1),
            "speedup": round(t1 / t2, 3)}


def bench_append(timer):
    """pkv_append in bulk: rows written to random distinct slots of a large
    cache (a prefill chunk's worth of rows per sequence, many sequences), and
    the decode step's shape (one row per sequence, 256 sequences)."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    Hkv, bs, D = 8, 16, 128
    nb = 16384
    desc = pkv.CacheDesc(nb, Hkv, bs, D, pkv.BF16)
    kc = torch.zeros(desc.cache_shape(), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    g = np.random.default_rng(23)
    res = {}
    for label, T, contiguous in (("random_slots", 65536, False), ("chunk_runs", 65536, True),
                                 ("decode_step", 256, False)):
        if contiguous:   # whole blocks in order: 512-token chunks of 128 sequences
            blocks = g.permutation(nb)[:T // bs]
            slots = (blocks[:, None] * bs + np.arange(bs)[None, :]).reshape(-1)
        else:
            slots = g.permutation(nb * bs)[:T]
        sl = torch.tensor(slots.astype(np.int32), device="cuda")
        k = torch.randn((T, Hkv, D), device="cuda").to(torch.bfloat16)
        v = torch.randn((T, Hkv, D), device="cuda").to(torch.bfloat16)
        t = float(np.median(timer.per_call(
            lambda: pkv.append(k, v, sl, kc, vc, desc), 30)))
        nbytes = 2 * T * Hkv * D * 2 * 2          # K and V rows read, and written
        res[label] = {"rows": T, "ms_per_call": round(1e3 * t, 4),
                      "GBps_read_plus_write": round(nbytes / t / 1e9, 1),
                      "frac_of_hbm_peak": round(nbytes / t / 1e9 / HBM_PEAK_GBS, 4)}
        if T <= 4096:
            # A call this small is shorter than its host-side launch path:
            # also time 64 calls captured in one HIP graph and replayed.
            n_rep = 64
            st = torch.cuda.Stream()
            with torch.cuda.stream(st):
                pkv.append(k, v, sl, kc, vc, desc)
            torch.cuda.synchronize()
            graph = torch.cuda.CUDAGraph()
            with torch.cuda.graph(graph, stream=st):
                for _ in range(n_rep):
                    pkv.append(k, v, sl, kc, vc, desc)
            tg = timer.amortized(graph.replay, 10, warmup=2) / n_rep
            res[label].update({"ms_per_call_graph_replay": round(1e3 * tg, 4),
                               "GBps_graph_replay": round(nbytes / tg / 1e9, 1),
                               "note": "ms_per_call: each call event-timed alone (host "
                                       "launch path included); graph replay: 64 calls back "
                                       "to back on the device"})
    res["workload"] = ("pkv_append: rows [T][8][128] bf16 into a 16384-block cache, slots random "
                       "and distinct, or whole blocks in order (prefill chunks), or one row per "
                       "sequence for 256 sequences (a decode step)")
    return res


def bench_block_copy(timer):
    """pkv_copy_blocks: copy-on-write style copies inside one cache, and a
    sequence's blocks swapped out to pinned host memory and back."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    Hkv, bs, D = 8, 16, 128
    nb = 16384                                   # 512 MiB per tensor
    desc = pkv.CacheDesc(nb, Hkv, bs, D, pkv.BF16)
    kc = torch.zeros(desc.cache_shape(), dtype=torch.bfloat16, device="cuda")
    vc = torch.zeros_like(kc)
    g = np.random.default_rng(17)
    perm = g.permutation(nb)
    n = 4096
    src = torch.tensor(perm[:n].astype(np.int32), device="cuda")
    dst = torch.tensor(perm[n:2 * n].astype(np.int32), device="cuda")
    blk = Hkv * bs * D * 2 * 2                   # K + V bytes of one block
    t = float(np.median(timer.per_call(
        lambda: pkv.copy_blocks(kc, vc, desc, kc, vc, desc, src, dst), 20)))
    res = {"workload": f"pkv_copy_blocks: {n} random block pairs in one cache of {nb} "
                       "blocks (8 KV heads x 16 x 128 bf16)",
           "ms_per_call": round(1e3 * t, 4),
           "hbm_GBps_read_plus_write": round(2 * n * blk / t / 1e9, 1),
           "frac_of_hbm_peak": round(2 * n * blk / t / 1e9 / HBM_PEAK_GBS, 4)}
    # Swap: one 8192-token sequence (512 blocks) out to pinned host and back.
    ns = 512
    hdesc = pkv.CacheDesc(ns, Hkv, bs, D, pkv.BF16)
    hk = torch.zeros(hdesc.cache_shape(), dtype=torch.bfloat16).pin_memory()
    hv = torch.zeros_like(hk).pin_memory()
    sids = torch.tensor(perm[:ns].astype(np.int32), device="cuda")
    hids = torch.arange(ns, dtype=torch.int32, device="cuda")
    t_out = float(np.median(timer.per_call(
        lambda: pkv.copy_blocks(kc, vc, desc, hk, hv, hdesc, sids, hids), 10)))
    t_in = float(np.median(timer.per_call(
        lambda: pkv.copy_blocks(hk, hv, hdesc, kc, vc, desc, hids, sids), 10)))
    res["swap"] = {"blocks": ns, "bytes": ns * blk,
                   "out_ms": round(1e3 * t_out, 4), "out_GBps": round(ns * blk / t_out / 1e9, 1),
                   "in_ms": round(1e3 * t_in, 4), "in_GBps": round(ns * blk / t_in / 1e9, 1),
                   "note": "kernel reads/writes pinned host memory directly over PCIe"}
    return res


def bench_prefix_ttft(timer):
    """TTFT proxy for prefix caching: the attention work of admitting one
    2560-token prompt (2048 shared + 512 own) in 512-token prefill chunks,
    cold (every chunk computed) vs with the 2048-token prefix served from
    the prefix cache (one chunk).  Appends of the computed chunks included."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    import synth
    from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows
    Hq, Hkv, D, bs, C, P = 64, 8, 128, 16, 512, 2048
    scale = 1.0 / np.sqrt(D)
    total = P + C
    g = synth.rng(46, synth.S_LENS)
    tok_shared = g.integers(0, 32000, size=P)
    tok_a = np.concatenate([tok_shared, g.integers(0, 32000, size=C)])
    tok_b = np.concatenate([tok_shared, g.integers(0, 32000, size=C)])
    k = synth.normal(synth.rng(46, synth.S_K), (total, Hkv, D), "bf16")
    v = synth.normal(synth.rng(46, synth.S_V), (total, Hkv, D), "bf16")
    q = synth.normal(synth.rng(46, synth.S_Q), (C, Hq, D), "bf16")
    cache = PagedCache(1024, Hkv, bs, D, pkv.BF16, pool_seed=4601)
    # Request A arrives cold and is registered; B shares its 2048-token prefix.
    cache.admit_cached(0, tok_a)
    cache.extend(0, k, v)
    cache.register(0, tok_a)
    reused = cache.admit_cached(1, tok_b)
    cache.extend(1, k[reused:], v[reused:])
    dq = to_device_rows(q, pkv.BF16, "cuda")
    qs = torch.tensor([0, C], dtype=torch.int32, device="cuda")
    out = torch.empty((C, Hq, D), dtype=torch.float32, device="cuda")
    dk = to_device_rows(k, pkv.BF16, "cuda")
    dv = to_device_rows(v, pkv.BF16, "cuda")
    slots_a = torch.tensor(np.concatenate([
        [b * bs + o for o in range(bs)] for b in cache.seqs.block_ids(0)])[:total].astype(
            np.int32), device="cuda")
    tab_a, _, _ = cache.tables([0])
    tab_b, lens_b, mx_b = cache.tables([1])
    lens_chunks = [torch.tensor([C * (i + 1)], dtype=torch.int32, device="cuda")
                   for i in range(total // C)]
    bb = cache.seqs.block_ids(1)
    slots_b = torch.tensor(np.array([bb[p // bs] * bs + p % bs for p in range(reused, total)],
                                    dtype=np.int32), device="cuda")

    pws = PrefillWorkspace().get(1, Hq, C, cache.desc)

    def cold():
        for i in range(total // C):
            lo = i * C
            pkv.append(dk[lo:lo + C], dv[lo:lo + C], slots_a[lo:lo + C], cache.k_cache,
                       cache.v_cache, cache.desc)
            pkv.prefill_chunk(dq, qs, cache.k_cache, cache.v_cache, tab_a, lens_chunks[i],
                              scale, out, cache.desc, C, C * (i + 1), workspace=pws)

    def warm():
        pkv.append(dk[reused:], dv[reused:], slots_b, cache.k_cache, cache.v_cache, cache.desc)
        pkv.prefill_chunk(dq, qs, cache.k_cache, cache.v_cache, tab_b, lens_b, scale, out,
                          cache.desc, C, mx_b, workspace=pws)
    t_cold = float(np.median(timer.per_call(cold, 10)))
    t_warm = float(np.median(timer.per_call(warm, 10)))
    return {"workload": "prefix cache TTFT proxy: one 2560-token prompt (2048-token shared "
                        "system prompt + 512 own), 512-token chunks, 64q/8kv, d128, bf16",
            "tokens_reused": int(reused),
            "cold_ms": round(1e3 * t_cold, 4),
            "cached_ms": round(1e3 * t_warm, 4),
            "ttft_reduction": round(1.0 - t_warm / t_cold, 4),
            "note": "attention + KV append only (no model layers); the page's ~50% TTFT "
                    "figure is for a whole model"}


def bench_sched(steps=300, warm=60):
    """The token-budget step scheduler driving the kernels: synthetic
    arrivals (Poisson, 0.25 requests per step; prompts U[512,4096], outputs
    U[64,256]), Llama-70B-shaped heads, 16-token blocks.  Each step appends
    the planned rows, runs pkv_prefill_chunk over the chunks and pkv_decode
    over the decode tokens.  Chunked (budget 2048, 512-token chunks) and
    unchunked (whole prompts, budget 4096 + decode) runs see the same
    arrivals.  Per step: GPU time of its kernels (HIP events); per request:
    TTFT = GPU time from the start of its arrival step to the end of the step
    that completes its prompt."""
    import torch
    import paged_kv_cache_indirected_amd as pkv
    from paged_kv_cache_indirected_amd.paged import PagedCache
    Hq, Hkv, D, bs = 64, 8, 128, 16
    scale = 1.0 / np.sqrt(D)
    g = np.random.default_rng(2024)
    arrivals = g.poisson(0.25, size=steps)
    lens = [(int(g.integers(512, 4097)), int(g.integers(64, 257))) for _ in range(int(arrivals.sum()))]
    rows = torch.randn((8192, Hkv, D), device="cuda").to(torch.bfloat16)
    qrows = torch.randn((8192, Hq, D), device="cuda").to(torch.bfloat16)
    out = {}
    for label, budget, chunk in (("chunked_512", 2048, 512), ("unchunked", 4096 + 64, 4096)):
        cache = PagedCache(12288, Hkv, bs, D, pkv.BF16, pool_seed=7)
        sc = pkv.Sched(cache.pool, cache.seqs, budget, chunk, max_running=64)
        ws = torch.zeros(pkv.decode_workspace_bytes(64, Hq, 8192, cache.desc), dtype=torch.uint8,
                         device="cuda")
        pout = torch.empty((budget, Hq, D), dtype=torch.float32, device="cuda")
        dout = torch.empty((64, Hq, D), dtype=torch.float32, device="cuda")
        pwsp = PrefillWorkspace()
        step_ms, arrive, ttft, clock, decoded, nreq = [], {}, [], 0.0, 0, 0
        for st in range(steps):
            for _ in range(int(arrivals[st])):
                sc.submit(nreq, *lens[nreq])
                arrive[nreq] = clock
                nreq += 1
            p = sc.step()
            slots = np.concatenate([p["chunk_slots"], p["decode_slots"]]).astype(np.int32)
            n = len(slots)
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            if len(p["chunk_ids"]):
                ptab, plens, pmx = cache.tables(list(p["chunk_ids"]))
                qs = torch.from_numpy(np.concatenate([[0], np.cumsum(p["chunk_len"])])
                                      .astype(np.int32)).cuda()
            if len(p["decode_ids"]):
                dtab, dlens, dmx = cache.tables(list(p["decode_ids"]))
            sl = torch.from_numpy(slots).cuda()
            pws = (pwsp.get(len(p["chunk_ids"]), Hq, int(p["chunk_len"].max()), cache.desc)
                   if len(p["chunk_ids"]) else None)
            e0.record()
            if n:
                pkv.append(rows[:n], rows[:n], sl, cache.k_cache, cache.v_cache, cache.desc)
            if len(p["chunk_ids"]):
                T = int(p["chunk_len"].sum())
                pkv.prefill_chunk(qrows[:T], qs, cache.k_cache, cache.v_cache, ptab, plens, scale,
                                  pout[:T], cache.desc, int(p["chunk_len"].max()), pmx,
                                  workspace=pws)
            if len(p["decode_ids"]):
                B = len(p["decode_ids"])
                pkv.decode(qrows[:B], cache.k_cache, cache.v_cache, dtab, dlens, scale, dout[:B],
                           cache.desc, dmx, workspace=ws)
            e1.record()
            torch.cuda.synchronize()
            ms = e0.elapsed_time(e1)
            clock += ms
            if st >= warm:
                step_ms.append(ms)
                decoded += len(p["decode_ids"])
                for rid in p["first_ids"]:
                    ttft.append(clock - arrive[int(rid)])
        sm = np.array(step_ms)
        tt = np.array(ttft) if ttft else np.zeros(1)
        out[label] = {"token_budget": budget, "chunk_tokens": chunk,
                      "step_ms_p50": round(float(np.percentile(sm, 50)), 3),
                      "step_ms_p90": round(float(np.percentile(sm, 90)), 3),
                      "step_ms_p99": round(float(np.percentile(sm, 99)), 3),
                      "step_ms_max": round(float(sm.max()), 3),
                      "ttft_ms_mean": round(float(tt.mean()), 3),
                      "ttft_ms_p90": round(float(np.percentile(tt, 90)), 3),
                      "first_tokens": len(ttft),
                      "decode_tokens_per_s": round(decoded / (sm.sum() * 1e-3), 1),
                      "running_at_end": sc.num_running, "waiting_at_end": sc.num_waiting}
        del cache, sc
        torch.cuda.empty_cache()
    out["workload"] = ("step scheduler: Poisson 0.25 req/step, prompts U[512,4096], outputs "
                       "U[64,256], 64q/8kv, d128, bf16, block 16, max 64 running; steps "
                       f"{warm}..{steps} timed (GPU time of each step's kernels)")
    return out


def probe_copy(nbytes=1 << 30, reps=3):
    """Run only the plain copy probe (nbytes read + nbytes written per call),
    so that a hardware-counter run sees a kernel of known traffic."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_indirected_amd", "libpkv_probe.so"))
    P = ctypes.c_void_p
    lib.pkv_probe_copy.argtypes = [P, P, ctypes.c_size_t, ctypes.c_int, P]
    src = torch.zeros(nbytes // 2, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    st = torch.cuda.current_stream().cuda_stream
    for _ in range(reps):
        lib.pkv_probe_copy(src.data_ptr(), dst.data_ptr(), nbytes // 16, 4096, st)
    torch.cuda.synchronize()
    print(json.dumps({"probe_copy_bytes": nbytes, "reps": reps}))


def probe_coissue(iters=20000, reps=3):
    """Matrix-core work beside vector work on one SIMD (pkv_probe_coissue):
    256 workgroups of 8 waves, waves w and w + 4 on one SIMD; each mode
    timed with HIP events on the launch stream, reps times, alternating."""
    import torch
    lib = ctypes.CDLL(os.path.join(ROOT, "paged_kv_cache_indirected_amd", "libpkv_probe.so"))
    P = ctypes.c_void_p
    lib.pkv_probe_coissue.argtypes = [P, ctypes.c_int, ctypes.c_int, ctypes.c_int, P]
    grid = 256
    out = torch.empty(grid * 512, dtype=torch.float32, device="cuda")
    st = torch.cuda.current_stream()
    names = ["mfma_waves_beside_fma_waves", "mfma_waves_alone", "fma_waves_alone",
             "one_wave_interleaved_1_mfma_3_fma"]
    times = {n: [] for n in names}
    for _ in range(reps):
        for mode, n in enumerate(names):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(st)
            rc = lib.pkv_probe_coissue(out.data_ptr(), iters, mode, grid, st.cuda_stream)
            e1.record(st)
            e1.synchronize()
            if rc != 0:
                raise RuntimeError(f"pkv_probe_coissue: {rc}")
            times[n].append(e0.elapsed_time(e1))
    print(json.dumps({"probe": "coissue", "iters": iters, "workgroups": grid,
                      "per_iteration": "8 v_mfma_f32_16x16x32_bf16 per MFMA wave, 24 fp32 FMA "
                                       "per FMA wave",
                      "ms": {n: [round(t, 3) for t in v] for n, v in times.items()}}))


def _pmc_per_dispatch(csv_path, name_part, counter):
    import csv
    vals = {}
    for r in csv.DictReader(open(csv_path)):
        if name_part in r["Kernel_Name"] and r["Counter_Name"] == counter:
            vals[r["Dispatch_Id"]] = vals.get(r["Dispatch_Id"], 0.0) + float(r["Counter_Value"])
    return [vals[k] for k in sorted(vals, key=int)]


def pmc_summary(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv, out_path, copy_bytes,
                kv_bytes):
    """HBM bytes per decode call from FETCH_SIZE / WRITE_SIZE runs (KiB per
    dispatch), each scaled by what the same counter reads for the copy probe
    of known size.  Steady-state dispatches only (the first of each kernel
    is dropped)."""
    fk = _pmc_per_dispatch(fetch_csv, "k_decode", "FETCH_SIZE")[1:]
    fm = _pmc_per_dispatch(fetch_csv, "k_merge", "FETCH_SIZE")[1:]
    wk = _pmc_per_dispatch(write_csv, "k_decode", "WRITE_SIZE")[1:]
    wm = _pmc_per_dispatch(write_csv, "k_merge", "WRITE_SIZE")[1:]
    cf = _pmc_per_dispatch(copy_fetch_csv, "k_copy", "FETCH_SIZE")
    cw = _pmc_per_dispatch(copy_write_csv, "k_copy", "WRITE_SIZE")
    sf = copy_bytes / (1024.0 * float(np.median(cf)))
    sw = copy_bytes / (1024.0 * float(np.median(cw)))
    fetch = 1024.0 * sf * (float(np.mean(fk)) + float(np.mean(fm)))
    write = 1024.0 * sw * (float(np.mean(wk)) + float(np.mean(wm)))
    rec = {
        "kernel": "pkv_decode call on the Llama-70B-shaped batch (k_decode + k_merge)",
        "decode_hip_sha256": hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest(),
        "fetch_KiB_per_dispatch": {"k_decode": float(np.mean(fk)), "k_merge": float(np.mean(fm))},
        "write_KiB_per_dispatch": {"k_decode": float(np.mean(wk)), "k_merge": float(np.mean(wm))},
        "copy_probe": {"bytes_each_way": copy_bytes, "fetch_KiB": float(np.median(cf)),
                       "write_KiB": float(np.median(cw)), "fetch_scale": sf, "write_scale": sw},
        "hbm_fetch_bytes_per_call": fetch,
        "hbm_write_bytes_per_call": write,
        "hbm_bytes_per_call": fetch + write,
        "algorithmic_bytes_per_call": kv_bytes,
        "traffic_over_algorithmic": (fetch + write) / kv_bytes,
    }
    with open(out_path, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def _pmc_calls(csv_path, counter, kernels, skip=1):
    """Per-call sums of a counter over the listed kernels (KiB): dispatch
    i of each kernel belongs to call i; the first `skip` calls (warm-up,
    cold caches) are dropped."""
    per = [_pmc_per_dispatch(csv_path, k, counter) for k in kernels]
    n = min(len(x) for x in per)
    return [sum(x[i] for x in per) for i in range(skip, n)]


def _copy_scale(copy_csv, counter, nbytes=1 << 30):
    return nbytes / (1024.0 * float(np.median(_pmc_per_dispatch(copy_csv, "k_copy", counter))))


def pmc_summary_indirection(id_csv, sh_csv, copy_fetch_csv):
    """FETCH_SIZE per decode call (k_decode + k_merge) for the identity and
    the shuffled placement, scaled by the copy probe's factor."""
    import synth
    b = synth.cfg2()
    sf = _copy_scale(copy_fetch_csv, "FETCH_SIZE")
    ident = 1024.0 * sf * float(np.mean(_pmc_calls(id_csv, "FETCH_SIZE", ["k_decode", "k_merge"])))
    shuf = 1024.0 * sf * float(np.mean(_pmc_calls(sh_csv, "FETCH_SIZE", ["k_decode", "k_merge"])))
    rec = {"kernel": "pkv_decode call on the Llama-70B-shaped batch (k_decode + k_merge), "
                     "identity vs shuffled block placement",
           "decode_hip_sha256": hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest(),
           "fetch_scale": sf,
           "identity_fetch_bytes_per_call": ident, "shuffled_fetch_bytes_per_call": shuf,
           "algorithmic_bytes_per_call": float(b.lens.sum()) * kv_row_bytes(b.shape)}
    with open(PMC_INDIRECTION_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def pmc_summary_cfg4(fetch_csv, write_csv, copy_fetch_csv, copy_write_csv):
    """HBM bytes per call of the prefix-sharing workload by counter: the
    plain decode (k_decode + k_merge, the calls before the cascade's first
    prefill-kernel dispatch) and the cascade decode (suffix k_decode +
    k_merge, prefix k_prefill, k_merge_states)."""
    import csv as _csv
    import synth
    sf = _copy_scale(copy_fetch_csv, "FETCH_SIZE")
    sw = _copy_scale(copy_write_csv, "WRITE_SIZE")

    def split(path, counter):
        rows = {}
        for r in _csv.DictReader(open(path)):
            if r["Counter_Name"] == counter:
                d = int(r["Dispatch_Id"])
                rows.setdefault(d, [r["Kernel_Name"], 0.0])[1] += float(r["Counter_Value"])
        order = sorted(rows)
        kind = [("dec" if "k_decode" in rows[d][0] else "mrg" if "k_merge<" in rows[d][0] else
                 "pf" if "k_prefill" in rows[d][0] else "ms" if "k_merge_states" in rows[d][0]
                 else "other") for d in order]
        val = [rows[d][1] for d in order]
        # A cascade call is the suffix k_decode + k_merge, the prefix
        # k_prefill and k_merge_states, enqueued in that order; a plain
        # call is a k_decode + k_merge pair with no k_prefill after it.
        plain, casc = [], []
        for i in range(len(order)):
            if kind[i] == "ms" and i >= 3 and kind[i - 3:i] == ["dec", "mrg", "pf"]:
                casc.append(sum(val[i - 3:i + 1]))
            elif (kind[i] == "dec" and i + 1 < len(order) and kind[i + 1] == "mrg" and
                  (i + 2 >= len(order) or kind[i + 2] != "pf")):
                plain.append(val[i] + val[i + 1])
        return float(np.mean(plain[3:])), float(np.mean(casc[3:]))
    pf, cf = split(fetch_csv, "FETCH_SIZE")
    pw, cw = split(write_csv, "WRITE_SIZE")
    b = synth.cfg4()
    row = kv_row_bytes(b.shape)
    rec = {"kernel": "prefix-sharing decode, 128 sequences on one 2048-token prefix: plain "
                     "pkv_decode (k_decode + k_merge) and pkv_decode_cascade (k_decode + k_merge "
                     "+ k_prefill + k_merge_states)",
           "decode_hip_sha256": hashlib.sha256(open(DECODE_SRC, "rb").read()).hexdigest(),
           "fetch_scale": sf, "write_scale": sw,
           "plain_hbm_bytes_per_call": 1024.0 * (sf * pf + sw * pw),
           "cascade_hbm_bytes_per_call": 1024.0 * (sf * cf + sw * cw),
           "plain_fetch_bytes_per_call": 1024.0 * sf * pf,
           "cascade_fetch_bytes_per_call": 1024.0 * sf * cf,
           "logical_kv_bytes": float(b.lens.sum()) * row,
           "unique_kv_bytes": float(b.prefix_len + (b.lens - b.prefix_len).sum()) * row}
    with open(PMC_CFG4_FILE, "w") as f:
        json.dump(rec, f, indent=1)
    print(json.dumps(rec))


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--copies", type=int, default=4)
    ap.add_argument("--splits", type=int, default=0,
                    help="decode workgroups per KV head (0: library choice)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--headline-only", action="store_true",
                    help="skip the other workloads and the probes")
    ap.add_argument("--only", choices=["continuous_batching", "prefix_sharing",
                                       "chunked_prefill_mixed", "append", "block_copy",
                                       "prefix_cache_ttft", "step_scheduler",
                                       "decode_batch_sweep"],
                    help="run one secondary workload alone (for profiling) and print its JSON")
    ap.add_argument("--probe-coissue", action="store_true",
                    help="time matrix-core work beside vector work on one SIMD and exit")
    ap.add_argument("--probe-copy", action="store_true",
                    help="run only the copy probe (for hardware-counter scaling)")
    ap.add_argument("--pmc-summary", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                       "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn counter CSVs into the committed per-call traffic summary")
    ap.add_argument("--indirection-pmc", choices=["identity", "shuffled"],
                    help="run only the Llama-70B-shaped decode call on one placement "
                         "(for a hardware-counter run)")
    ap.add_argument("--pmc-summary-indirection", nargs=3,
                    metavar=("IDENTITY_FETCH_CSV", "SHUFFLED_FETCH_CSV", "COPY_FETCH_CSV"),
                    help="turn the two placements' FETCH_SIZE CSVs into the committed summary")
    ap.add_argument("--pmc-summary-cfg4", nargs=4,
                    metavar=("FETCH_CSV", "WRITE_CSV", "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="turn counter CSVs of '--only prefix_sharing' into the committed summary")
    args = ap.parse_args()
    if args.pmc_summary_indirection:
        pmc_summary_indirection(*args.pmc_summary_indirection)
        return
    if args.pmc_summary_cfg4:
        pmc_summary_cfg4(*args.pmc_summary_cfg4)
        return
    if args.pmc_summary:
        import synth
        b = synth.cfg2()
        pmc_summary(*args.pmc_summary, PMC_FILE, 1 << 30,
                    float(b.lens.sum()) * kv_row_bytes(b.shape))
        return
    if args.probe_coissue:
        probe_coissue()
        return
    if args.probe_copy:
        probe_copy()
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU only; --gpus {args.gpus} is not supported: the "
              "paged-KV path here runs on one GPU (no sharding, no collectives)", file=sys.stderr)
        sys.exit(2)

    import torch
    import paged_kv_cache_indirected_amd as pkv
    import synth

    torch.cuda.set_device(0)
    timer = Timer()
    if args.only:
        fns = {"continuous_batching": lambda: bench_cfg3(timer, 10, args.splits),
               "prefix_sharing": lambda: bench_cfg4(timer, args.splits),
               "chunked_prefill_mixed": lambda: bench_cfg5(timer, args.splits),
               "append": lambda: bench_append(timer),
               "block_copy": lambda: bench_block_copy(timer),
               "prefix_cache_ttft": lambda: bench_prefix_ttft(timer),
               "step_scheduler": lambda: bench_sched(),
               "decode_batch_sweep": lambda: bench_decode_sweep(timer)}
        print(json.dumps({args.only: fns[args.only]()}), flush=True)
        return
    batch = synth.cfg2()
    sh = batch.shape
    if args.indirection_pmc:
        if args.indirection_pmc == "identity":
            sts = identity_states(batch, args.copies)
        else:
            sts = [paged_state(batch, batch.pool_seed + 7919 * r) for r in range(args.copies)]
        mx = max(s["max_len"] for s in sts)
        ws = workspace(batch.B, sh.Hq, mx, sts[0]["cache"].desc, args.splits)
        o = torch.empty((batch.B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
        for i in range(args.warmup + args.steps):
            s = sts[i % len(sts)]
            c = s["cache"]
            pkv.decode(s["q"], c.k_cache, c.v_cache, s["tables"], s["lens"], sh.scale, o, c.desc,
                       mx, workspace=ws, num_splits=args.splits)
        torch.cuda.synchronize()
        print(json.dumps({"indirection_pmc": args.indirection_pmc, "calls": args.steps,
                          "warmup": args.warmup}))
        return
    log(f"[bench] building {args.copies} paged copies of the Llama-70B-shaped batch "
        f"(B={batch.B}, sum L={int(batch.lens.sum())}, pool={batch.pool_blocks} blocks)")
    states = [paged_state(batch, batch.pool_seed + 7919 * r) for r in range(args.copies)]
    out = torch.empty((batch.B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    desc = states[0]["cache"].desc
    max_len = max(s["max_len"] for s in states)
    ws = workspace(batch.B, sh.Hq, max_len, desc, args.splits)
    splits = args.splits or pkv.decode_num_splits(batch.B, sh.Hq, max_len, desc)
    q = states[0]["q"]

    def decode_call(s):
        c = s["cache"]
        pkv.decode(q, c.k_cache, c.v_cache, s["tables"], s["lens"], sh.scale, out, c.desc,
                   max_len, workspace=ws, num_splits=args.splits)

    def step(i):
        # The decode step in one call: append of each sequence's new token
        # fused with the decode (pkv_append_decode).
        s = states[i % len(states)]
        c = s["cache"]
        pkv.append_decode(s["k_new"], s["v_new"], s["slots"], q, c.k_cache, c.v_cache,
                          s["tables"], s["lens"], sh.scale, out, c.desc, max_len, workspace=ws,
                          num_splits=args.splits)

    def step_two_calls(i):
        s = states[i % len(states)]
        c = s["cache"]
        pkv.append(s["k_new"], s["v_new"], s["slots"], c.k_cache, c.v_cache, c.desc)
        decode_call(s)

    def run_steps(fn):
        for i in range(args.warmup):
            fn(i)
        torch.cuda.synchronize()
        t0 = torch.cuda.Event(enable_timing=True)
        t1 = torch.cuda.Event(enable_timing=True)
        t0.record()
        for i in range(args.steps):
            fn(i)
        t1.record()
        torch.cuda.synchronize()
        return t0.elapsed_time(t1) / args.steps

    # Both ways of running the step are timed; the headline is the faster.
    ms_step_fused = run_steps(step)
    ms_step_two = run_steps(step_two_calls)
    ms_step = min(ms_step_fused, ms_step_two)
    step_kind = "pkv_append_decode" if ms_step_fused <= ms_step_two else "pkv_append + pkv_decode"
    # The fused step captured once per paged copy in a HIP graph and replayed,
    # as a serving loop would run it (reported beside the eager headline).
    graphs = []
    for i in range(len(states)):
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            step(i)
        graphs.append(g)
    ms_step_graph = run_steps(lambda i: graphs[i % len(graphs)].replay())
    del graphs

    # The decode call alone (split kernel + merge kernel), each bracketed by
    # events on the launch stream.
    it = [0]

    def one_decode():
        decode_call(states[it[0] % len(states)])
        it[0] += 1
    dec_s = timer.per_call(one_decode, args.steps)
    dec_avg = float(dec_s.mean())

    kv_bytes = float(batch.lens.sum()) * kv_row_bytes(sh)
    gbs_step = kv_bytes / (ms_step * 1e-3) / 1e9
    gbs_dec = kv_bytes / dec_avg / 1e9
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
            "step_calls": step_kind,
            "global_batch": batch.B,
            "context_tokens": int(batch.lens.sum()),
            "pool_copies_rotated": len(states),
            "splits_per_kv_head": splits,
        },
        "pct_of_hbm_peak": round(100.0 * gbs_step / HBM_PEAK_GBS, 2),
        "ms_per_step_append_then_decode": round(ms_step_two, 5),
        "ms_per_step_fused_append_decode": round(ms_step_fused, 5),
        "ms_per_step_fused_hip_graph_replay": round(ms_step_graph, 5),
        "seq_steps_per_s": round(batch.B / (ms_step * 1e-3), 1),
        "roofline": {
            "bound": "hbm",
            "kernel": "pkv_decode call (k_decode split pass + k_merge)",
            "achieved": round(gbs_dec, 1),
            "peak": HBM_PEAK_GBS,
            "unit": "GB/s",
            "frac": round(gbs_dec / HBM_PEAK_GBS, 4),
            "traffic": pmc_traffic(kv_bytes),
            "algorithmic_bytes_per_launch": int(kv_bytes),
            "avg_launch_ms": round(1e3 * dec_avg, 5),
            "p10_ms": round(1e3 * float(np.percentile(dec_s, 10)), 5),
            "p90_ms": round(1e3 * float(np.percentile(dec_s, 90)), 5),
            "side_bytes_per_launch": decode_side_bytes(batch.lens, sh, splits),
        },
    }
    side = res["roofline"]["side_bytes_per_launch"]
    if res["roofline"]["traffic"]:
        res["roofline"]["traffic_over_algorithmic_plus_side"] = round(
            res["roofline"]["traffic"] / (kv_bytes + side["total"]), 4)
    if not args.headline_only:
        log("[bench] probes")
        probes, plib, sink = bench_probes(timer)
        probes["paged_tile_read_GBps"] = bench_tile_probe(plib, sink, states, sh, kv_bytes, timer)
        probes["paged_tile_note"] = ("the decode's 4 KiB (block, KV head) tiles of the same "
                                     "shuffled pools, K and V, no arithmetic: one workgroup per "
                                     "CU, each wave a contiguous run of the tile list (the 8 KV "
                                     "heads of a block back to back; 1, 2 or 4 heads per run read "
                                     "alike), two tiles in flight")
        res["roofline"]["achievable_probes"] = probes
        res["roofline"]["frac_of_paged_tile_probe"] = round(
            gbs_dec / probes["paged_tile_read_GBps"], 4)
        log("[bench] cost of indirection (identity vs shuffled placement)")
        indirection = bench_indirection(timer, batch, states, args.splits)
        del states
        torch.cuda.empty_cache()
        log("[bench] step metadata (pinned host -> device)")
        metadata = bench_metadata(timer, batch)
        torch.cuda.empty_cache()
        log("[bench] continuous batching")
        wl = {"indirection": indirection, "metadata_h2d": metadata}
        wl["continuous_batching"] = bench_cfg3(timer, 10, args.splits)
        torch.cuda.empty_cache()
        log("[bench] prefix sharing")
        wl["prefix_sharing"] = bench_cfg4(timer, args.splits)
        torch.cuda.empty_cache()
        log("[bench] chunked prefill + decode")
        wl["chunked_prefill_mixed"] = bench_cfg5(timer, args.splits)
        torch.cuda.empty_cache()
        log("[bench] decode batch-size sweep")
        wl["decode_batch_sweep"] = bench_decode_sweep(timer)
        torch.cuda.empty_cache()
        log("[bench] append")
        wl["append"] = bench_append(timer)
        torch.cuda.empty_cache()
        log("[bench] block copy and swap")
        wl["block_copy"] = bench_block_copy(timer)
        torch.cuda.empty_cache()
        log("[bench] prefix cache TTFT proxy")
        wl["prefix_cache_ttft"] = bench_prefix_ttft(timer)
        torch.cuda.empty_cache()
        log("[bench] step scheduler")
        wl["step_scheduler"] = bench_sched()
        res["workloads"] = wl
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle baseline")
        res["cpu_baseline"] = cpu_baseline(batch)
        log("[bench] timing the CPU oracle on one thread (tiny and Llama-70B-shaped steps)")
        res["cpu_baseline"]["one_thread"] = {"tiny_f32_d64": cpu_single_thread(synth.cfg1()),
                                             "llama70b_shaped": cpu_single_thread(batch, 1.0)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
