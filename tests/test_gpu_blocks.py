"""Block copy, fork with copy-on-write, and prefix-cache reuse on the GPU.

pkv_copy_blocks is compared bit for bit with the oracle's copy over whole
cache images (every bit pattern, NaNs included, must survive).  Fork +
copy-on-write and prefix-cache admission are checked end to end: each
sequence's decode or prefill output against the oracle's attention over that
sequence's logical rows (the rows it was given, in order), so a block that
was shared when it should have been copied, or copied from the wrong place,
shows up as a wrong output.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_indirected_amd as pkv
import synth
from harness import DT, TOL, max_err, run_decode, run_prefill, sample_rows, say
from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows

pytestmark = pytest.mark.gpu

_BITS = {"f32": (np.uint32, np.int32, torch.int32), "bf16": (np.uint16, np.int16, torch.int16)}


def _random_image(g, shape, dtype):
    u, s, _ = _BITS[dtype]
    return g.integers(0, np.iinfo(u).max, size=shape, dtype=u, endpoint=True).view(s)


def _to_dev(img, dtype, pinned=False):
    t = torch.from_numpy(img.copy())
    t = t.pin_memory() if pinned else t.cuda()
    return t.view(torch.float32 if dtype == "f32" else torch.bfloat16)


def _to_host(t, dtype):
    return t.view(_BITS[dtype][2]).cpu().numpy()


def _ids(a):
    return torch.tensor(np.asarray(a, dtype=np.int32)).cuda()


@pytest.mark.parametrize("dtype,D,bs,Hkv", [("f32", 64, 16, 8), ("bf16", 128, 16, 8),
                                            ("bf16", 128, 32, 1), ("bf16", 64, 32, 2),
                                            ("f32", 128, 32, 4)])
def test_copy_blocks_in_place_bitexact(dtype, D, bs, Hkv):
    g = synth.rng(41, 0, D, bs, Hkv)
    nb = 97
    shape = (nb, Hkv, bs, D)
    kimg, vimg = _random_image(g, shape, dtype), _random_image(g, shape, dtype)
    perm = g.permutation(nb)
    src = perm[:30].astype(np.int32)
    dst = perm[30:60].astype(np.int32)
    src[[3, 11]] = [-1, nb + 5]           # skipped pairs: source outside the cache
    dst[[7, 19]] = [nb, -2]               # skipped pairs: destination outside the cache
    say(f"[copy] in place {dtype} D={D} bs={bs} Hkv={Hkv} pairs={len(src)}")
    desc = pkv.CacheDesc(nb, Hkv, bs, D, DT[dtype])
    kc, vc = _to_dev(kimg, dtype), _to_dev(vimg, dtype)
    pkv.copy_blocks(kc, vc, desc, kc, vc, desc, _ids(src), _ids(dst))
    torch.cuda.synchronize()
    oracle.copy_blocks(kimg, vimg, kimg, vimg, src, dst)
    assert np.array_equal(_to_host(kc, dtype), kimg)
    assert np.array_equal(_to_host(vc, dtype), vimg)


def test_copy_blocks_swap_out_to_pinned_host_and_back():
    # Device cache -> pinned host swap area (another cache of the same block
    # shape, different size) -> back into other device blocks.
    dtype, D, bs, Hkv = "bf16", 128, 16, 8
    g = synth.rng(42, 0)
    nb, nh = 64, 20
    kimg = _random_image(g, (nb, Hkv, bs, D), dtype)
    vimg = _random_image(g, (nb, Hkv, bs, D), dtype)
    hk = np.zeros((nh, Hkv, bs, D), dtype=np.int16)
    hv = np.zeros_like(hk)
    dd = pkv.CacheDesc(nb, Hkv, bs, D, DT[dtype])
    hd = pkv.CacheDesc(nh, Hkv, bs, D, DT[dtype])
    kc, vc = _to_dev(kimg, dtype), _to_dev(vimg, dtype)
    hkc, hvc = _to_dev(hk, dtype, pinned=True), _to_dev(hv, dtype, pinned=True)
    out_src = g.permutation(nb)[:12].astype(np.int32)
    out_dst = g.permutation(nh)[:12].astype(np.int32)
    say("[copy] swap out 12 blocks to pinned host, swap back in")
    pkv.copy_blocks(kc, vc, dd, hkc, hvc, hd, _ids(out_src), _ids(out_dst))
    torch.cuda.synchronize()
    oracle.copy_blocks(kimg, vimg, hk, hv, out_src, out_dst)
    assert np.array_equal(hkc.view(torch.int16).numpy(), hk)
    assert np.array_equal(hvc.view(torch.int16).numpy(), hv)
    back_dst = np.setdiff1d(np.arange(nb), out_src)[:12].astype(np.int32)
    pkv.copy_blocks(hkc, hvc, hd, kc, vc, dd, _ids(out_dst), _ids(back_dst))
    torch.cuda.synchronize()
    oracle.copy_blocks(hk, hv, kimg, vimg, out_dst, back_dst)
    assert np.array_equal(_to_host(kc, dtype), kimg)
    assert np.array_equal(_to_host(vc, dtype), vimg)


def test_copy_blocks_many_pairs():
    # 3000 pairs of 32 KiB blocks in one launch (24,000 workgroups).
    dtype, D, bs, Hkv = "bf16", 128, 16, 8
    g = synth.rng(43, 0)
    nb = 6144
    kimg = _random_image(g, (nb, Hkv, bs, D), dtype)
    vimg = _random_image(g, (nb, Hkv, bs, D), dtype)
    perm = g.permutation(nb)
    src, dst = perm[:3000].astype(np.int32), perm[3000:6000].astype(np.int32)
    say(f"[copy] {len(src)} pairs, nb={nb}")
    desc = pkv.CacheDesc(nb, Hkv, bs, D, DT[dtype])
    kc, vc = _to_dev(kimg, dtype), _to_dev(vimg, dtype)
    pkv.copy_blocks(kc, vc, desc, kc, vc, desc, _ids(src), _ids(dst))
    torch.cuda.synchronize()
    oracle.copy_blocks(kimg, vimg, kimg, vimg, src, dst)
    assert np.array_equal(_to_host(kc, dtype), kimg)
    assert np.array_equal(_to_host(vc, dtype), vimg)


# --------------------------------------------------------------------------
# Fork + copy-on-write, end to end through decode.

@pytest.mark.parametrize("dtype,D,bs", [("bf16", 128, 16), ("f32", 64, 32), ("bf16", 64, 32)])
def test_fork_cow_decode_matches_oracle(dtype, D, bs):
    Hq, Hkv = 16, 2
    sh = synth.Shape(Hq=Hq, Hkv=Hkv, D=D, dtype=dtype, block_size=bs, scale=1.0 / np.sqrt(D))
    g = synth.rng(44, 0, D, bs)
    L0 = 3 * bs + 5                                   # the forked block is partially filled
    tails = [1, bs, 2 * bs + 3, 7]                    # each branch's own tokens
    base_k = synth.normal(synth.rng(44, synth.S_K, D, bs), (L0, Hkv, D), dtype)
    base_v = synth.normal(synth.rng(44, synth.S_V, D, bs), (L0, Hkv, D), dtype)
    tail_k = [synth.normal(synth.rng(44, synth.S_K, D, bs, i + 1), (t, Hkv, D), dtype)
              for i, t in enumerate(tails)]
    tail_v = [synth.normal(synth.rng(44, synth.S_V, D, bs, i + 1), (t, Hkv, D), dtype)
              for i, t in enumerate(tails)]
    nb = 64
    say(f"[cow] fork decode {dtype} D={D} bs={bs} L0={L0} tails={tails}")
    cache = PagedCache(nb, Hkv, bs, D, DT[dtype], pool_seed=int(g.integers(1, 2**40)))
    cache.add_sequences([0], [L0], base_k, base_v)
    for b in (1, 2, 3):
        cache.fork(b, 0)
    # Decode-style steps: one token per still-growing branch per step.
    n_copies = 0
    for step in range(max(tails)):
        ids = [b for b in range(4) if step < tails[b]]
        rk = np.stack([tail_k[b][step] for b in ids])
        rv = np.stack([tail_v[b][step] for b in ids])
        _, copies = cache.step_cow(ids, rk, rv)
        n_copies += len(copies)
    # Four holders of the partial block, all in the first step's batch:
    # three copies, the last holder keeps the original.
    assert n_copies == 3
    lens = np.array([L0 + t for t in tails], dtype=np.int64)
    k = np.concatenate([np.concatenate([base_k, tail_k[b]]) for b in range(4)])
    v = np.concatenate([np.concatenate([base_v, tail_v[b]]) for b in range(4)])
    q = synth.normal(synth.rng(44, synth.S_Q, D, bs), (4, Hq, D), dtype)
    tables, dlens, max_len = cache.tables(range(4))
    out = run_decode(cache, to_device_rows(q, DT[dtype], cache.device), tables, dlens, max_len,
                     sh.scale)
    ref = oracle.decode(q, k, v, lens, sh.scale)
    err = max_err(out, ref)
    say(f"[cow] max err {err:.3g}")
    assert err <= TOL[dtype]
    # The shared full blocks were never copied.
    ids0 = cache.seqs.block_ids(0)
    for b in (1, 2, 3):
        assert cache.seqs.block_ids(b)[:3] == ids0[:3]


# --------------------------------------------------------------------------
# Prefix cache, end to end through prefill.

def test_prefix_cache_reuse_prefill_matches_oracle():
    # A 2048-token shared prompt ("Prefix caching"), llama-70B-shaped heads.
    Hq, Hkv, D, bs, dtype = 64, 8, 128, 16, "bf16"
    scale = 1.0 / np.sqrt(D)
    P = 2048
    g = synth.rng(45, synth.S_LENS)
    shared_tok = g.integers(0, 32000, size=P + 5)
    tok_a = np.concatenate([shared_tok, g.integers(0, 32000, size=40)])
    tok_b = np.concatenate([shared_tok, g.integers(0, 32000, size=300)])
    rows_a = len(tok_a)
    ka = synth.normal(synth.rng(45, synth.S_K, 0), (rows_a, Hkv, D), dtype)
    va = synth.normal(synth.rng(45, synth.S_V, 0), (rows_a, Hkv, D), dtype)
    # B's KV equals A's over the common prefix (it depends only on the prefix).
    nb_own = len(tok_b) - len(shared_tok)
    kb = np.concatenate([ka[:len(shared_tok)],
                         synth.normal(synth.rng(45, synth.S_K, 1), (nb_own, Hkv, D), dtype)])
    vb = np.concatenate([va[:len(shared_tok)],
                         synth.normal(synth.rng(45, synth.S_V, 1), (nb_own, Hkv, D), dtype)])
    cache = PagedCache(512, Hkv, bs, D, DT[dtype], pool_seed=451)
    assert cache.admit_cached(0, tok_a) == 0
    cache.extend(0, ka, va)
    cache.register(0, tok_a)
    reused = cache.admit_cached(1, tok_b)
    assert reused == oracle.reusable_prefix_tokens(list(tok_b), [list(tok_a)], bs) == P
    assert cache.seqs.block_ids(1) == cache.seqs.block_ids(0)[:P // bs]
    cache.extend(1, kb[reused:], vb[reused:])
    C = len(tok_b) - reused
    say(f"[prefix] reused {reused} of {len(tok_b)} tokens; prefill chunk {C}")
    q = synth.normal(synth.rng(45, synth.S_Q, 0), (C, Hq, D), dtype)
    tables, lens, max_len = cache.tables([1])
    qs = torch.tensor([0, C], dtype=torch.int32, device=cache.device)
    out = run_prefill(cache, to_device_rows(q, DT[dtype], cache.device), qs, tables, lens,
                      max_len, scale, C)
    rows = sample_rows(C, Hq, 768, 46)
    ref = oracle.prefill(q, np.array([0, C]), kb, vb, np.array([len(tok_b)]), scale, rows=rows)
    err = max_err(out, ref, pairs=rows)
    say(f"[prefix] max err {err:.3g}")
    assert err <= TOL[dtype]
    # After both finish, the cached blocks stay reusable for a third request.
    cache.register(1, tok_b)
    cache.release(0)
    cache.release(1)
    assert cache.pool.num_cached == (len(tok_a) // bs) + (len(tok_b) // bs) - P // bs
    expect = oracle.reusable_prefix_tokens(list(tok_b), [list(tok_a), list(tok_b)], bs)
    assert cache.admit_cached(2, tok_b) == expect == (len(tok_b) - 1) // bs * bs


# --------------------------------------------------------------------------
# Preemption by swap, end to end: swap out, let other work overwrite every
# free device block, swap back in, decode again.

@pytest.mark.parametrize("dtype,D,bs", [("bf16", 128, 16), ("f32", 64, 32)])
def test_swap_roundtrip_decode_bitwise(dtype, D, bs):
    from harness import decode_state
    b = synth.custom_decode(47, [40, 300, 17, 129, 1, 64], Hq=16, Hkv=2, D=D, dtype=dtype,
                            block_size=bs)
    say(f"[swap] {dtype} D={D} bs={bs} lens={list(b.lens)}")
    cache, q, tab, lens, mx = decode_state(b)
    before = run_decode(cache, q, tab, lens, mx, b.shape.scale)
    cache.attach_swap(64)
    moved = cache.swap_out(1) + cache.swap_out(3)
    assert moved and cache.seqs.is_swapped(1)
    # Another sequence takes every free device block and fills it with junk.
    nfree = cache.pool.num_free
    junk = synth.normal(synth.rng(47, 9), (nfree * bs, 2, D), dtype)
    cache.seqs.add(99)
    cache.extend(99, junk, junk)
    cache.release(99)
    cache.swap_in(1)
    cache.swap_in(3)
    tab2, lens2, mx2 = cache.tables(range(b.B))
    after = run_decode(cache, q, tab2, lens2, mx2, b.shape.scale)
    assert torch.equal(before, after)
    ref = oracle.decode(b.q, b.k, b.v, b.lens, b.shape.scale)
    assert max_err(after, ref) <= TOL[dtype]
