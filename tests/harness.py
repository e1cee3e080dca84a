"""Shared helpers of the GPU tests: build paged state from a synthetic batch
through the product API, run the kernels, and compare against the oracle."""
from __future__ import annotations

import sys

import numpy as np
import torch

import paged_kv_cache_indirected_amd as pkv
import synth
from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows

DT = {"f32": pkv.F32, "bf16": pkv.BF16}
TOL = {"f32": 1e-5, "bf16": 2e-3}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def decode_state(batch: synth.DecodeBatch, pool_seed=None, poison=None, share_prefix=True,
                 pool_blocks=None):
    """Load every sequence's rows but the last through the pool and
    pkv_append, then run the step's bookkeeping + append of the last row
    (one token per sequence).  Returns (cache, q, tables, lens, max_len)."""
    sh = batch.shape
    seed = batch.pool_seed if pool_seed is None else pool_seed
    nb = pool_blocks or batch.pool_blocks
    if batch.prefix_len and not share_prefix:
        nb = nb + batch.B * (batch.prefix_len // sh.block_size)
    cache = PagedCache(nb, sh.Hkv, sh.block_size, sh.D, DT[sh.dtype], pool_seed=seed,
                       poison=poison)
    st = batch.seq_start()
    ids = list(range(batch.B))
    if batch.prefix_len and share_prefix:
        P = batch.prefix_len
        cache.add_sequences([-1], [P], batch.k[:P], batch.v[:P])
        for b in ids:
            cache.add_shared(b, -1, P)
            lo, hi = st[b] + P, st[b + 1] - 1
            cache.extend(b, batch.k[lo:hi], batch.v[lo:hi])
    else:
        rows_k = np.concatenate([batch.k[st[b]:st[b + 1] - 1] for b in ids])
        rows_v = np.concatenate([batch.v[st[b]:st[b + 1] - 1] for b in ids])
        cache.add_sequences(ids, batch.lens - 1, rows_k, rows_v)
    # The step: one new token per sequence (bookkeeping, then pkv_append).
    slots = cache.seqs.append_batch(ids)
    last = st[1:] - 1
    cache.write(slots, batch.k[last], batch.v[last])
    tables, lens, max_len = cache.tables(ids)
    q = to_device_rows(batch.q, DT[sh.dtype], cache.device)
    return cache, q, tables, lens, max_len


def step_state(batch, pool_seed=None):
    """Cache holding every row but each sequence's last; the step's slots
    from the pool; the last rows as device tensors.  Returns (cache, slots,
    k_new, v_new, q, tables, lens, max_len)."""
    sh = batch.shape
    st = batch.seq_start()
    ids = list(range(batch.B))
    cache = PagedCache(batch.pool_blocks, sh.Hkv, sh.block_size, sh.D, DT[sh.dtype],
                       pool_seed=batch.pool_seed if pool_seed is None else pool_seed)
    cache.add_sequences(ids, batch.lens - 1,
                        np.concatenate([batch.k[st[b]:st[b + 1] - 1] for b in ids]),
                        np.concatenate([batch.v[st[b]:st[b + 1] - 1] for b in ids]))
    slots = cache.seqs.append_batch(ids)
    tables, lens, mx = cache.tables(ids)
    last = st[1:] - 1
    return (cache, torch.from_numpy(slots).to(cache.device),
            to_device_rows(batch.k[last], DT[sh.dtype], cache.device),
            to_device_rows(batch.v[last], DT[sh.dtype], cache.device),
            to_device_rows(batch.q, DT[sh.dtype], cache.device), tables, lens, mx)


def run_decode(cache: PagedCache, q, tables, lens, max_len, scale, out_dtype=torch.float32,
               num_splits=0):
    B, Hq, D = q.shape
    out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    nbytes = pkv.decode_workspace_bytes(B, Hq, max_len, cache.desc, num_splits)
    ws = torch.zeros(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    pkv.decode(q, cache.k_cache, cache.v_cache, tables, lens, scale, out, cache.desc, max_len,
               workspace=ws, num_splits=num_splits)
    torch.cuda.synchronize()
    return out


def sample_pairs(B, Hq, n, seed):
    g = np.random.default_rng(seed)
    if B * Hq <= n:
        return None
    flat = g.choice(B * Hq, size=n, replace=False)
    return np.stack([flat // Hq, flat % Hq], axis=1).astype(np.int32)


def max_err(out: torch.Tensor, ref: np.ndarray, pairs=None) -> float:
    o = out.float().cpu().numpy().astype(np.float64)
    if pairs is None:
        return float(np.max(np.abs(o - ref))) if o.size else 0.0
    e = 0.0
    for b, h in pairs:
        e = max(e, float(np.max(np.abs(o[b, h] - ref[b, h]))))
    return e


def prefill_state(batch: synth.PrefillBatch, pool_seed=None, poison=None):
    """Append every sequence's prior rows and its chunk through the pool and
    pkv_append (the chunk is in the cache before the prefill call).  Returns
    (cache, q, query_start, tables, lens, max_len)."""
    sh = batch.shape
    seed = batch.pool_seed if pool_seed is None else pool_seed
    cache = PagedCache(batch.pool_blocks, sh.Hkv, sh.block_size, sh.D, DT[sh.dtype],
                       pool_seed=seed, poison=poison)
    ids = list(range(len(batch.chunk)))
    cache.add_sequences(ids, batch.lens, batch.k, batch.v)
    tables, lens, max_len = cache.tables(ids)
    q = to_device_rows(batch.q, DT[sh.dtype], cache.device)
    qs = torch.from_numpy(batch.query_start.astype(np.int32)).to(cache.device)
    return cache, q, qs, tables, lens, max_len


def prefill_workspace(S, Hq, max_query_len, desc, device="cuda"):
    """The workspace pkv_prefill_chunk asks for (key-split states), or None."""
    n = pkv.prefill_workspace_bytes(S, Hq, max_query_len, desc)
    return torch.empty(n, dtype=torch.uint8, device=device) if n else None


def run_prefill(cache: PagedCache, q, qs, tables, lens, max_len, scale, max_query_len,
                out_dtype=torch.float32, split=True):
    """pkv_prefill_chunk; split=False passes no workspace (one pass per
    workgroup over all its keys), split=True the workspace it asks for (the
    library then splits the keys where the grid is short)."""
    out = torch.empty(tuple(q.shape), dtype=out_dtype, device=q.device)
    ws = prefill_workspace(int(qs.numel()) - 1, int(q.shape[1]), max_query_len, cache.desc,
                           q.device) if split else None
    pkv.prefill_chunk(q, qs, cache.k_cache, cache.v_cache, tables, lens, scale, out, cache.desc,
                      max_query_len, max_len, workspace=ws)
    torch.cuda.synchronize()
    return out


def sample_rows(T, Hq, n, seed):
    """n distinct (token row, head) pairs, or None for all when T*Hq <= n."""
    g = np.random.default_rng(seed)
    if T * Hq <= n:
        return None
    flat = g.choice(T * Hq, size=n, replace=False)
    return np.stack([flat // Hq, flat % Hq], axis=1).astype(np.int32)
