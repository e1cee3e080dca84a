"""Slot-mapped append on the GPU, bit-exact against the oracle's slot writes
over the whole cache image, untouched (poisoned) bytes included."""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_indirected_amd as pkv
import synth
from harness import DT, say
from paged_kv_cache_indirected_amd.paged import PagedCache, to_device_rows

pytestmark = pytest.mark.gpu


def _host_cache(cache: PagedCache) -> np.ndarray:
    t = cache.k_cache
    return (t.view(torch.int32) if t.dtype == torch.float32 else t.view(torch.int16)).cpu().numpy()


def _image(cache):
    kc = _host_cache(cache)
    vc = (cache.v_cache.view(torch.int32) if cache.v_cache.dtype == torch.float32
          else cache.v_cache.view(torch.int16)).cpu().numpy()
    return kc, vc


def _row(img: np.ndarray, blk: int, head: int, t: int, which: int) -> np.ndarray:
    """Row of token offset t in tile (blk, head) of a cache image
    [num_blocks][Hkv][bs][D], through the oracle's tile layout."""
    _, _, bs, D = img.shape
    flat = img[blk, head].reshape(-1)
    return np.array([flat[oracle.tile_index(t, d, bs, D, img.dtype.itemsize)[which]]
                     for d in range(D)], dtype=img.dtype)


def _raw(rows, dtype):
    return rows.view(np.int32) if dtype == "f32" else rows.view(np.int16)


def _check_batch(batch: synth.DecodeBatch):
    sh = batch.shape
    say(f"[append] {batch.name} B={batch.B} rows={int(batch.lens.sum())}")
    cache = PagedCache(batch.pool_blocks, sh.Hkv, sh.block_size, sh.D, DT[sh.dtype],
                       pool_seed=batch.pool_seed)
    slots = cache.add_sequences(range(batch.B), batch.lens, batch.k, batch.v)
    torch.cuda.synchronize()
    kc, vc = _image(cache)
    pois = synth.POISON_F32 if sh.dtype == "f32" else synth.POISON_BF16
    dt = np.int32 if sh.dtype == "f32" else np.int16
    ek = np.full(kc.shape, np.array(pois).astype(np.uint32 if sh.dtype == "f32" else np.uint16)
                 .view(dt), dtype=dt)
    ev = ek.copy()
    oracle.append(_raw(batch.k, sh.dtype), _raw(batch.v, sh.dtype), slots, ek, ev, sh.block_size)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


def test_cfg1_append_bitexact():
    _check_batch(synth.cfg1())


def test_cfg3_append_bitexact_subset():
    _check_batch(synth.cfg3_initial(B=48))


def test_cfg2_append_bitexact_subset():
    _check_batch(synth.cfg2(B=6))


@pytest.mark.parametrize("dtype,D", [("f32", 128), ("bf16", 64)])
def test_other_row_widths(dtype, D):
    _check_batch(synth.custom_decode(21, [3, 40, 17], Hq=4, Hkv=4, D=D, dtype=dtype,
                                     block_size=32))


def test_negative_and_out_of_range_slots_write_nothing():
    sh_nb, H, bs, D = 8, 2, 16, 128
    cache = PagedCache(sh_nb, H, bs, D, pkv.BF16)
    g = np.random.default_rng(0)
    k = g.integers(0, 2**16, size=(5, H, D), dtype=np.uint16)
    v = g.integers(0, 2**16, size=(5, H, D), dtype=np.uint16)
    slots = np.array([3, -1, sh_nb * bs + 5, 127, -7], dtype=np.int32)
    cache.write(slots, k, v)
    torch.cuda.synchronize()
    kc, vc = _image(cache)
    ek = np.full(kc.shape, np.int16(0x7FC0), dtype=np.int16)
    ev = ek.copy()
    ok = np.where((slots >= 0) & (slots < sh_nb * bs), slots, -1)
    oracle.append(k.view(np.int16), v.view(np.int16), ok, ek, ev, bs)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


def _mixed_slots(g, nslots, T):
    """T slot entries: runs of consecutive slots (random start, so some are
    4-aligned at a 4-aligned row and some are not), lone random slots and -1
    padding, all distinct."""
    used, out = set(), []
    while len(out) < T:
        kind = g.integers(0, 4)
        if kind == 0:
            out.extend([-1] * int(g.integers(1, 4)))
            continue
        n = 1 if kind == 1 else int(g.integers(2, 41))
        s0 = int(g.integers(0, nslots - n))
        run = list(range(s0, s0 + n))
        if any(x in used for x in run):
            continue
        used.update(run)
        out.extend(run)
    return np.array(out[:T], dtype=np.int32)


@pytest.mark.parametrize("dtype,D,bs", [("bf16", 128, 16), ("bf16", 128, 32), ("bf16", 64, 16),
                                        ("f32", 128, 16), ("f32", 64, 32)])
def test_run_groups_and_row_groups_mixed(dtype, D, bs):
    """Groups of 4 rows whose slots are 4 consecutive, 4-aligned slots take
    the whole-group path; every other group (misaligned or broken runs,
    padding, the ragged last group) goes row by row.  Both must equal the
    oracle's slot writes over the whole image."""
    nb, H, T = 48, 2, 203
    g = np.random.default_rng([7, D, bs, len(dtype)])
    slots = _mixed_slots(g, nb * bs, T)
    say(f"[append mixed] {dtype} D={D} bs={bs} T={T} runs+rows")
    dt_np = np.int32 if dtype == "f32" else np.int16
    k = g.integers(-2**15, 2**15, size=(T, H, D)).astype(dt_np)
    v = g.integers(-2**15, 2**15, size=(T, H, D)).astype(dt_np)
    cache = PagedCache(nb, H, bs, D, DT[dtype])
    kd = torch.from_numpy(k.view(np.float32) if dtype == "f32" else k).cuda()
    vd = torch.from_numpy(v.view(np.float32) if dtype == "f32" else v).cuda()
    if dtype == "bf16":
        kd, vd = kd.view(torch.bfloat16), vd.view(torch.bfloat16)
    pkv.append(kd, vd, torch.from_numpy(slots).cuda(), cache.k_cache, cache.v_cache, cache.desc)
    torch.cuda.synchronize()
    kc, vc = _image(cache)
    pois = synth.POISON_F32 if dtype == "f32" else synth.POISON_BF16
    ek = np.full(kc.shape, np.array(pois).astype(np.uint32 if dtype == "f32" else np.uint16)
                 .view(dt_np), dtype=dt_np)
    ev = ek.copy()
    oracle.append(k, v, slots, ek, ev, bs)
    assert np.array_equal(kc, ek) and np.array_equal(vc, ev)


def test_append_is_idempotent_and_overwrites():
    cache = PagedCache(4, 1, 16, 64, pkv.F32)
    g = np.random.default_rng(1)
    k1 = g.standard_normal((3, 1, 64), dtype=np.float32)
    k2 = g.standard_normal((3, 1, 64), dtype=np.float32)
    s = np.array([0, 17, 63], dtype=np.int32)
    cache.write(s, k1, k1)
    cache.write(s, k2, k2)
    cache.write(s, k2, k2)
    torch.cuda.synchronize()
    kc = cache.k_cache.cpu().numpy()
    vc = cache.v_cache.cpu().numpy()
    for i, slot in enumerate(s):
        assert np.array_equal(_row(kc, slot // 16, 0, slot % 16, 0), k2[i, 0])
        assert np.array_equal(_row(vc, slot // 16, 0, slot % 16, 1), k2[i, 0])


def test_logical_readback_after_appends_is_the_concatenation():
    # After n appends, reading the cache through the block table gives the
    # sequence rows in order ("The KV cache": append each step).
    b = synth.custom_decode(22, [70, 5], Hq=2, Hkv=2, D=64, dtype="bf16", block_size=16)
    cache = PagedCache(b.pool_blocks, 2, 16, 64, pkv.BF16, pool_seed=b.pool_seed)
    st = b.seq_start()
    for s in range(b.B):
        cache.seqs.add(s)
    for t in range(int(b.lens.max())):
        for s in range(b.B):
            if t < b.lens[s]:
                cache.extend(s, b.k[st[s] + t:st[s] + t + 1], b.v[st[s] + t:st[s] + t + 1])
    torch.cuda.synchronize()
    kc = cache.k_cache.view(torch.int16).cpu().numpy()
    vc = cache.v_cache.view(torch.int16).cpu().numpy()
    for s in range(b.B):
        ids = cache.seqs.block_ids(s)
        for t in range(int(b.lens[s])):
            for h in range(2):
                assert np.array_equal(_row(kc, ids[t // 16], h, t % 16, 0),
                                      b.k[st[s] + t, h].view(np.int16))
                assert np.array_equal(_row(vc, ids[t // 16], h, t % 16, 1),
                                      b.v[st[s] + t, h].view(np.int16))
