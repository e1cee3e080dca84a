"""Cascade decode over a shared prefix (pkv_decode_cascade) against the
oracle's attention over each sequence's logical rows (prefix rows followed by
its own), and against the plain split decode over the concatenated block
lists."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_indirected_amd as pkv
import synth
from harness import DT, TOL, decode_state, max_err, run_decode, sample_pairs, say
from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows

pytestmark = pytest.mark.gpu


def _cascade(cache, q, prefix_ids, P, tables, lens, scale, out_dtype=torch.float32):
    nbp = P // cache.desc.block_size
    B, Hq, D = q.shape
    tab_s = tables[:, nbp:].contiguous() if tables.shape[1] > nbp else \
        torch.full((B, 1), -1, dtype=torch.int32, device=q.device)
    lens_s = (lens - P).to(torch.int32).contiguous()
    mx = int(lens_s.max().item()) if B else 0
    out = torch.empty((B, Hq, D), dtype=out_dtype, device=q.device)
    pb = torch.tensor(prefix_ids[:nbp], dtype=torch.int32, device=q.device) if nbp else None
    nbytes = pkv.decode_cascade_workspace_bytes(B, Hq, P, mx, cache.desc)
    ws = torch.empty(max(nbytes, 1), dtype=torch.uint8, device=q.device)
    ws.fill_(0xFF)                          # the workspace needs no initialisation
    pkv.decode_cascade(q, cache.k_cache, cache.v_cache, pb, P, tab_s, lens_s, scale, out,
                       cache.desc, mx, workspace=ws)
    torch.cuda.synchronize()
    return out


def test_cfg4_cascade_matches_oracle_and_plain_decode():
    b = synth.cfg4()
    P = b.prefix_len
    say(f"[cascade] cfg4 B={b.B} prefix={P}")
    cache, q, tab, lens, mx = decode_state(b)
    out = _cascade(cache, q, cache.seqs.block_ids(-1), P, tab, lens, b.shape.scale)
    pairs = sample_pairs(b.B, b.shape.Hq, 512, 61)
    ref = oracle.decode(b.q, b.k, b.v, b.lens, b.shape.scale, pairs=pairs)
    err = max_err(out, ref, pairs)
    plain = run_decode(cache, q, tab, lens, mx, b.shape.scale)
    d = float((out - plain).abs().max())
    say(f"[cascade] cfg4 err {err:.3g}, |cascade - plain| {d:.3g}")
    assert err <= TOL["bf16"] and d <= TOL["bf16"]


def _shared_batch(seed, B, P, own, Hq, Hkv, D, bs):
    """Logical rows: P shared prefix rows, then own[b] rows per sequence."""
    sh = synth.Shape(Hq=Hq, Hkv=Hkv, D=D, dtype="bf16", block_size=bs, scale=1.0 / np.sqrt(D))
    pk = synth.normal(synth.rng(seed, synth.S_PREFIX, 0), (P, Hkv, D), "bf16")
    pv = synth.normal(synth.rng(seed, synth.S_PREFIX, 1), (P, Hkv, D), "bf16")
    ok = [synth.normal(synth.rng(seed, synth.S_K, i), (n, Hkv, D), "bf16") for i, n in enumerate(own)]
    ov = [synth.normal(synth.rng(seed, synth.S_V, i), (n, Hkv, D), "bf16") for i, n in enumerate(own)]
    q = synth.normal(synth.rng(seed, synth.S_Q), (B, Hq, D), "bf16")
    nb = P // bs + sum((n + bs - 1) // bs for n in own) + 8
    cache = PagedCache(nb, Hkv, bs, D, pkv.BF16, pool_seed=seed)
    if P:
        cache.add_sequences([-1], [P], pk, pv)
    for i, n in enumerate(own):
        if P:
            cache.add_shared(i, -1, P)
        else:
            cache.seqs.add(i)
        if n:
            cache.extend(i, ok[i], ov[i])
    tab, lens, _ = cache.tables(range(B))
    K = np.concatenate([np.concatenate([pk, ok[i]]) for i in range(B)])
    V = np.concatenate([np.concatenate([pv, ov[i]]) for i in range(B)])
    L = np.array([P + n for n in own])
    prefix_ids = cache.seqs.block_ids(-1) if P else []
    return sh, cache, q, tab, lens, K, V, L, prefix_ids


@pytest.mark.parametrize("B,P,own,G,D,bs", [
    (5, 16 * 7, [0, 1, 17, 40, 3], 8, 128, 16),
    (1, 32 * 3, [9], 4, 64, 32),
    (3, 0, [5, 70, 16], 8, 128, 16),
    (9, 16 * 33, [1] * 9, 1, 128, 16),
    (40, 16 * 64, list(range(40)), 8, 128, 16),
    (2, 32, [0, 0], 2, 64, 32),
    # More sequences than one decode launch holds (1024): the suffix
    # launches, each merging its own sequences, run beside the prefix pass.
    (1100, 16 * 4, [i % 5 for i in range(1100)], 1, 64, 16),
])
def test_cascade_shapes(B, P, own, G, D, bs):
    Hkv = 2
    sh, cache, q, tab, lens, K, V, L, pids = _shared_batch(62 + B, B, P, own, G * Hkv, Hkv, D, bs)
    say(f"[cascade] B={B} P={P} G={G} D={D} bs={bs}")
    out = _cascade(cache, to_device_rows(q, pkv.BF16, "cuda"), pids, P, tab, lens, sh.scale)
    ref = oracle.decode(q, K, V, L, sh.scale)
    err = max_err(out, ref)
    assert err <= TOL["bf16"], err


def test_cascade_bf16_output():
    sh, cache, q, tab, lens, K, V, L, pids = _shared_batch(70, 4, 64, [3, 30, 0, 11], 16, 2, 128, 16)
    out = _cascade(cache, to_device_rows(q, pkv.BF16, "cuda"), pids, 64, tab, lens, sh.scale,
                   out_dtype=torch.bfloat16)
    ref = oracle.decode(q, K, V, L, sh.scale)
    o = out.float().cpu().numpy()
    half_ulp = np.abs(ref) * 2.0 ** -9
    assert np.all(np.abs(o - ref) <= TOL["bf16"] + half_ulp)
