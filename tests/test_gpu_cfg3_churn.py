"""Continuous batching at its full shape on the GPU, every step against the
fp64 oracle ("LLM Inference: KV Cache, Batching & Scheduling", "Continuous
batching (Orca)": sequences leave and join at every step; "PagedAttention and
vLLM": a finished request's blocks go back to the pool at once and are
handed out again).

256 sequences, 64 query / 8 KV heads, head_dim 128, bf16, 32-token blocks,
log-normal contexts; ten steps, each appending one token per sequence and
decoding in one fused launch (pkv_append_decode), then 26 sequences finish
and are replaced by new ones of 16-128 tokens -- the same step sequence the
benchmark times.  The pool is sized so that, from the third step on, the
replacements and the growing sequences take blocks the finished ones left
behind, with their old contents still in them (the pool's free list is
first in, first out).  Each step compares 512
(sequence, head) rows with the oracle, two heads of every batch position.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_indirected_amd as pkv
import synth
from harness import TOL, max_err, say
from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows

pytestmark = pytest.mark.gpu

STEPS = 10


def test_cfg3_churn_steps_against_oracle():
    b0 = synth.cfg3_initial()
    sh = b0.shape
    B, bs = b0.B, sh.block_size
    st = b0.seq_start()
    pre = b0.lens - 1                         # tokens cached before step 1
    need0 = int(np.sum((pre + bs - 1) // bs))
    # Headroom for about one step of growth and replacements: after that the
    # free list's front is used up and blocks released by finished sequences
    # (returned to its back) are handed out again.
    num_blocks = need0 + 96
    say(f"[cfg3 churn] B={B} initial tokens={int(pre.sum())} blocks={num_blocks}")
    cache = PagedCache(num_blocks, sh.Hkv, bs, sh.D, pkv.BF16, pool_seed=b0.pool_seed)
    ids = list(range(B))
    # Each batch position's logical rows, as a list of row blocks in append
    # order (the oracle's input is their concatenation).
    shadow_k = [[b0.k[st[p]:st[p + 1] - 1]] for p in ids]
    shadow_v = [[b0.v[st[p]:st[p + 1] - 1]] for p in ids]
    cache.add_sequences(ids, pre, np.concatenate([c[0] for c in shadow_k]),
                        np.concatenate([c[0] for c in shadow_v]))
    del b0
    next_id = B
    stride = (8192 + 1 + STEPS + bs) // bs + 1
    out = torch.empty((B, sh.Hq, sh.D), dtype=torch.float32, device="cuda")
    ws = torch.empty(pkv.decode_workspace_bytes(B, sh.Hq, stride * bs, cache.desc),
                     dtype=torch.uint8, device="cuda")
    released, reused = set(), 0
    g = np.random.default_rng(31)
    for step in range(1, STEPS + 1):
        slots_np = cache.seqs.append_batch(ids)
        slots = torch.from_numpy(slots_np).to("cuda")
        kn, vn, qn = synth.cfg3_step_rows(step, B, sh)
        for p in range(B):
            shadow_k[p].append(kn[p:p + 1])
            shadow_v[p].append(vn[p:p + 1])
        held = {blk for p in ids for blk in cache.seqs.block_ids(p)}
        reused += len(held & released)
        tab, lens, mx = cache.tables(ids, stride)
        lens_np = np.array([sum(len(x) for x in c) for c in shadow_k], dtype=np.int64)
        assert np.array_equal(lens.cpu().numpy(), lens_np)
        out.fill_(float("nan"))
        pkv.append_decode(to_device_rows(kn, pkv.BF16, "cuda"), to_device_rows(vn, pkv.BF16, "cuda"),
                          slots, to_device_rows(qn, pkv.BF16, "cuda"), cache.k_cache,
                          cache.v_cache, tab, lens, sh.scale, out, cache.desc, mx, workspace=ws)
        torch.cuda.synchronize()
        # Two heads of every batch position.
        heads = np.stack([g.choice(sh.Hq, size=2, replace=False) for _ in range(B)])
        pairs = np.array([(p, h) for p in range(B) for h in heads[p]], dtype=np.int32)
        ref = oracle.decode(qn, np.concatenate([x for c in shadow_k for x in c]),
                            np.concatenate([x for c in shadow_v for x in c]), lens_np, sh.scale,
                            pairs=pairs)
        err = max_err(out, ref, pairs)
        say(f"  step {step}: tokens={int(lens_np.sum())} max abs err {err:.3e} "
            f"(blocks from finished sequences in use: {len(held & released)})")
        assert err <= TOL["bf16"], (step, err)
        # Churn: 26 sequences finish, their blocks go back to the pool, and
        # new sequences take their batch positions.
        ev = synth.cfg3_churn(step, B, sh)
        for i, pos in enumerate(ev.finished):
            released |= set(cache.seqs.block_ids(ids[pos]))
            cache.release(ids[pos])
            ids[pos] = next_id
            cache.add_sequences([next_id], [int(ev.new_lens[i])], ev.new_k[i], ev.new_v[i])
            shadow_k[pos] = [ev.new_k[i]]
            shadow_v[pos] = [ev.new_v[i]]
            next_id += 1
    assert reused > 0, "no block of a finished sequence was handed out again"
