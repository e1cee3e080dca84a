"""Paged decode on the GPU against the fp64 oracle, plus the invariants the
pages fix ("LLM Inference: KV Cache, Batching & Scheduling": blocks are mapped
not moved, shared prefix blocks hold what duplicated ones would).

Bars: max abs error 1e-5 (fp32 inputs) and 2e-3 (bf16 inputs) on fp32
output; bitwise equality for the placement, sharing, poison and determinism
invariants; exact V for a length-1 context.
"""
import numpy as np
import pytest
import torch

import oracle
import synth
from harness import TOL, decode_state, max_err, run_decode, sample_pairs, say, step_state

pytestmark = pytest.mark.gpu


def _check(batch, pairs=None, **kw):
    say(f"[decode] {batch.name} B={batch.B} maxL={int(batch.lens.max())} {kw}")
    cache, q, tab, lens, mx = decode_state(batch)
    out = run_decode(cache, q, tab, lens, mx, batch.shape.scale, **kw)
    ref = oracle.decode(batch.q, batch.k, batch.v, batch.lens, batch.shape.scale, pairs=pairs)
    err = max_err(out, ref, pairs)
    say(f"  max abs err {err:.3e}")
    assert err <= TOL[batch.shape.dtype], err
    return out


def test_cfg1_tiny_fp32():
    _check(synth.cfg1())


def test_cfg2_llama70b_shape_full():
    _check(synth.cfg2())


def test_cfg3_initial_sampled():
    b = synth.cfg3_initial()
    _check(b, pairs=sample_pairs(b.B, b.shape.Hq, 768, 3))


def test_cfg4_prefix_shared_sampled():
    b = synth.cfg4()
    _check(b, pairs=sample_pairs(b.B, b.shape.Hq, 512, 4))


def test_cfg5_decode_part_sampled():
    _, dec = synth.cfg5()
    _check(dec, pairs=sample_pairs(dec.B, dec.shape.Hq, 512, 5))


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_shape_sweep_ragged(dtype, D, bs, G):
    lens = [1, 2, bs - 1, bs, bs + 1, 4 * bs + 3, 300, 1000]
    b = synth.custom_decode(100 + G + D + bs, lens, Hq=2 * G, Hkv=2, D=D, dtype=dtype,
                            block_size=bs)
    _check(b)


def test_identity_vs_shuffled_placement_bitwise():
    b = synth.cfg2(B=8)
    outs = []
    for seed in (0, b.pool_seed, 12345):
        cache, q, tab, lens, mx = decode_state(b, pool_seed=seed)
        outs.append(run_decode(cache, q, tab, lens, mx, b.shape.scale))
    assert torch.equal(outs[0], outs[1]) and torch.equal(outs[0], outs[2])


def test_shared_prefix_equals_duplicated_bitwise():
    b = synth.cfg4(B=16)
    c1 = decode_state(b, share_prefix=True)
    c2 = decode_state(b, share_prefix=False)
    o1 = run_decode(*c1, b.shape.scale)
    o2 = run_decode(*c2, b.shape.scale)
    assert torch.equal(o1, o2)
    ref = oracle.decode(b.q, b.k, b.v, b.lens, b.shape.scale)
    assert max_err(o1, ref) <= TOL["bf16"]


def test_poison_does_not_leak_bitwise():
    b = synth.custom_decode(7, [5, 17, 33, 64, 250], Hq=16, Hkv=2, D=128, dtype="bf16",
                            block_size=16)
    o_nan = run_decode(*decode_state(b), b.shape.scale)
    o_zero = run_decode(*decode_state(b, poison=0x0000), b.shape.scale)
    o_big = run_decode(*decode_state(b, poison=0x7F7F), b.shape.scale)
    assert torch.isfinite(o_nan).all()
    assert torch.equal(o_nan, o_zero) and torch.equal(o_nan, o_big)


def test_split_count_independence():
    # One workgroup per KV head (every sequence whole, no merge) against
    # splits that cut sequences into up to hundreds of pieces.
    b = synth.cfg2(B=6)
    cache, q, tab, lens, mx = decode_state(b)
    base = run_decode(cache, q, tab, lens, mx, b.shape.scale, num_splits=1)
    ref = oracle.decode(b.q, b.k, b.v, b.lens, b.shape.scale)
    assert max_err(base, ref) <= TOL["bf16"]
    for ns in (2, 3, 17, 128, 1000, 0):
        o = run_decode(cache, q, tab, lens, mx, b.shape.scale, num_splits=ns)
        assert float((o - base).abs().max()) <= 1e-5, ns


def test_empty_and_tiny_sequences_between_long_ones():
    # Empty sequences inside the batch, and ranges that hold several whole
    # short sequences plus pieces of long ones.
    lens = [0, 3000, 1, 0, 17, 2000, 0, 33, 5, 0]
    b = synth.custom_decode(12, [max(L, 1) for L in lens], Hq=64, Hkv=8, D=128, dtype="bf16",
                            block_size=16)
    cache, q, tab, lens_d, mx = decode_state(b)
    for i, L in enumerate(lens):
        if L == 0:
            lens_d[i] = 0
    for ns in (1, 7, 64, 0):
        out = run_decode(cache, q, tab, lens_d, mx, b.shape.scale, num_splits=ns)
        for i, L in enumerate(lens):
            if L == 0:
                assert torch.count_nonzero(out[i]) == 0
        keep = [i for i, L in enumerate(lens) if L > 0]
        st = b.seq_start()
        kk = np.concatenate([b.k[st[i]:st[i + 1]] for i in keep])
        vv = np.concatenate([b.v[st[i]:st[i + 1]] for i in keep])
        ref = oracle.decode(b.q[keep], kk, vv, b.lens[keep], b.shape.scale)
        assert max_err(out[keep], ref) <= TOL["bf16"], ns


def test_batch_above_one_launch():
    # More sequences than one launch takes (1024): the call splits the batch.
    g = np.random.default_rng(13)
    lens = g.integers(1, 40, size=1100)
    b = synth.custom_decode(13, lens, Hq=8, Hkv=8, D=64, dtype="f32", block_size=16)
    cache, q, tab, lens_d, mx = decode_state(b)
    out = run_decode(cache, q, tab, lens_d, mx, b.shape.scale)
    ref = oracle.decode(b.q, b.k, b.v, b.lens, b.shape.scale)
    assert max_err(out, ref) <= TOL["f32"]


@pytest.mark.parametrize("B", [63, 64, 65, 257])
def test_batch_sizes_around_the_wave_width(B):
    # The block prefix sums are computed by each wave alone up to 64
    # sequences and by the whole workgroup above: both sides of the switch,
    # with empty sequences among them.
    g = np.random.default_rng([17, B])
    lens = g.integers(1, 200, size=B)
    b = synth.custom_decode(17 + B, lens, Hq=16, Hkv=2, D=128, dtype="bf16", block_size=16)
    cache, q, tab, lens_d, mx = decode_state(b)
    empty = [i for i in range(B) if i % 9 == 4]
    for i in empty:
        lens_d[i] = 0
    out = run_decode(cache, q, tab, lens_d, mx, b.shape.scale)
    for i in empty:
        assert torch.count_nonzero(out[i]) == 0
    keep = [i for i in range(B) if i % 9 != 4]
    st = b.seq_start()
    kk = np.concatenate([b.k[st[i]:st[i + 1]] for i in keep])
    vv = np.concatenate([b.v[st[i]:st[i + 1]] for i in keep])
    ref = oracle.decode(b.q[keep], kk, vv, b.lens[keep], b.shape.scale)
    assert max_err(out[keep], ref) <= TOL["bf16"]


def test_length_one_returns_v_exactly():
    for dtype in ("f32", "bf16"):
        b = synth.custom_decode(9, [1, 1, 1], Hq=16, Hkv=2, D=128, dtype=dtype, block_size=16)
        out = run_decode(*decode_state(b), b.shape.scale).cpu().numpy()
        v = b.v if dtype == "f32" else synth.bf16_to_f32(b.v)
        for s in range(3):
            for h in range(16):
                assert np.array_equal(out[s, h], v[s, h // 8])


def test_empty_context_gives_zeros():
    b = synth.custom_decode(10, [1, 40], Hq=8, Hkv=1, D=64, dtype="bf16", block_size=16)
    cache, q, tab, lens, mx = decode_state(b)
    lens[0] = 0
    out = run_decode(cache, q, tab, lens, mx, b.shape.scale)
    assert torch.count_nonzero(out[0]) == 0
    ref = oracle.decode(b.q[1:], b.k[1:], b.v[1:], b.lens[1:], b.shape.scale)
    assert max_err(out[1:], ref) <= TOL["bf16"]


def test_lengths_clamped_to_max_context_len():
    # A device length above max_context_len is clamped to it, a negative one
    # to 0 (empty context: zeros); the other sequences are unaffected.  The
    # longest sequence is the one raised past the bound, so that the clamp
    # lands on its true length.
    b = synth.cfg2(B=6)
    cache, q, tab, lens, mx = decode_state(b)
    i = int(np.argmax(b.lens))
    j = (i + 2) % b.B
    assert int(b.lens[i]) == mx
    lens[i] = mx + 37
    lens[j] = -5
    out = run_decode(cache, q, tab, lens, mx, b.shape.scale)
    assert torch.count_nonzero(out[j]) == 0
    keep = [s for s in range(b.B) if s != j]
    ref = oracle.decode(b.q, b.k, b.v, b.lens, b.shape.scale)
    err = max_err(out[keep], ref[keep])
    say(f"[decode] clamped lengths: max abs err {err:.3e}")
    assert err <= TOL["bf16"]


def test_bf16_output_rounding():
    b = synth.cfg2(B=4)
    cache, q, tab, lens, mx = decode_state(b)
    out = run_decode(cache, q, tab, lens, mx, b.shape.scale, out_dtype=torch.bfloat16)
    ref = oracle.decode(b.q, b.k, b.v, b.lens, b.shape.scale)
    o = out.float().cpu().numpy().astype(np.float64)
    half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 8)
    assert np.all(np.abs(o - ref) <= 2e-3 + half_ulp)


def test_repeat_is_bitwise_deterministic():
    b = synth.cfg2(B=8)
    st = decode_state(b)
    o1 = run_decode(*st, b.shape.scale)
    o2 = run_decode(*st, b.shape.scale)
    assert torch.equal(o1, o2)


def test_out_of_range_block_id_contributes_nothing():
    # A table entry outside the pool is a precondition violation that the
    # kernel's bounds check turns into "no contribution".
    b = synth.custom_decode(11, [64], Hq=8, Hkv=1, D=128, dtype="bf16", block_size=16)
    cache, q, tab, lens, mx = decode_state(b)
    tab[0, 1] = cache.desc.num_blocks + 100
    out = run_decode(cache, q, tab, lens, mx, b.shape.scale)
    keep = np.r_[0:16, 32:64]
    ref = oracle.decode(b.q, b.k[keep], b.v[keep], [48], b.shape.scale)
    assert max_err(out, ref) <= TOL["bf16"]


def test_workspace_reused_across_calls():
    # One workspace serves calls of different batches and split counts back
    # to back: nothing a call leaves in it changes the next call's result.
    import paged_kv_cache_indirected_amd as pkv
    b1 = synth.cfg2(B=6)
    b2 = synth.custom_decode(14, [700, 5, 1300], Hq=64, Hkv=8, D=128, dtype="bf16",
                             block_size=16)
    st1, st2 = decode_state(b1), decode_state(b2)
    ws = torch.zeros(pkv.decode_workspace_bytes(6, 64, 4096, st1[0].desc, 1000),
                     dtype=torch.uint8, device="cuda")
    r1 = oracle.decode(b1.q, b1.k, b1.v, b1.lens, b1.shape.scale)
    r2 = oracle.decode(b2.q, b2.k, b2.v, b2.lens, b2.shape.scale)
    for ns in (7, 64, 3, 1000, 0):
        for (cache, q, tab, lens, mx), ref in ((st1, r1), (st2, r2)):
            out = torch.empty(tuple(q.shape), dtype=torch.float32, device="cuda")
            pkv.decode(q, cache.k_cache, cache.v_cache, tab, lens, b1.shape.scale, out, cache.desc,
                       mx, workspace=ws, num_splits=ns)
            torch.cuda.synchronize()
            assert max_err(out, ref) <= TOL["bf16"], ns


@pytest.mark.parametrize("name", ["cfg1", "cfg2", "ragged-bs32-f32", "many-short"])
def test_append_decode_equals_append_then_decode_bitwise(name):
    import paged_kv_cache_indirected_amd as pkv
    splits = (0, 3)
    if name == "cfg1":
        b = synth.cfg1()
    elif name == "cfg2":
        b = synth.cfg2(B=8)
    elif name == "many-short":
        # 150 sequences of 1..40 tokens: with one workgroup per KV head it
        # holds the last block of every sequence, more new rows than it keeps
        # for the end of its range, so the rest are written at once.
        lens = np.random.default_rng(17).integers(1, 41, size=150)
        b = synth.custom_decode(17, lens.tolist(), Hq=16, Hkv=2, D=128, dtype="bf16",
                                block_size=16)
        splits = (0, 1, 3)
    else:
        b = synth.custom_decode(15, [1, 2, 31, 32, 33, 100], Hq=8, Hkv=2, D=128, dtype="f32",
                                block_size=32)
    say(f"[append_decode] {name}")
    cache, slots, kn, vn, q, tab, lens, mx = step_state(b)
    kc0, vc0 = cache.k_cache.clone(), cache.v_cache.clone()
    B, Hq, D = q.shape
    for ns in splits:
        ws = torch.zeros(pkv.decode_workspace_bytes(B, Hq, mx, cache.desc, ns), dtype=torch.uint8,
                         device="cuda")
        cache.k_cache.copy_(kc0)
        cache.v_cache.copy_(vc0)
        o1 = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        pkv.append(kn, vn, slots, cache.k_cache, cache.v_cache, cache.desc)
        pkv.decode(q, cache.k_cache, cache.v_cache, tab, lens, b.shape.scale, o1, cache.desc, mx,
                   workspace=ws, num_splits=ns)
        torch.cuda.synchronize()
        k1, v1 = cache.k_cache.clone(), cache.v_cache.clone()
        cache.k_cache.copy_(kc0)
        cache.v_cache.copy_(vc0)
        o2 = torch.empty_like(o1)
        pkv.append_decode(kn, vn, slots, q, cache.k_cache, cache.v_cache, tab, lens, b.shape.scale,
                          o2, cache.desc, mx, workspace=ws, num_splits=ns)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2)
        assert torch.equal(k1.view(torch.uint8), cache.k_cache.view(torch.uint8))
        assert torch.equal(v1.view(torch.uint8), cache.v_cache.view(torch.uint8))
    ref = oracle.decode(b.q, b.k, b.v, b.lens, b.shape.scale)
    assert max_err(o2, ref) <= TOL[b.shape.dtype]


def test_append_decode_skipped_slots_and_empty_sequences():
    # A negative slot appends nothing (position L-1 then comes from the
    # cache, written beforehand here); a sequence of length 0 still gets its
    # row written and a zero output.
    import paged_kv_cache_indirected_amd as pkv
    b = synth.custom_decode(16, [40, 1, 17, 300], Hq=16, Hkv=2, D=128, dtype="bf16",
                            block_size=16)
    cache, slots, kn, vn, q, tab, lens, mx = step_state(b)
    pkv.append(kn[:1], vn[:1], slots[:1], cache.k_cache, cache.v_cache, cache.desc)
    slots_f = slots.clone()
    slots_f[0] = -1
    lens[2] = 0
    torch.cuda.synchronize()
    kc0, vc0 = cache.k_cache.clone(), cache.v_cache.clone()
    B, Hq, D = q.shape
    ws = torch.zeros(pkv.decode_workspace_bytes(B, Hq, mx, cache.desc, 0), dtype=torch.uint8,
                     device="cuda")
    o2 = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
    pkv.append_decode(kn, vn, slots_f, q, cache.k_cache, cache.v_cache, tab, lens, b.shape.scale,
                      o2, cache.desc, mx, workspace=ws)
    torch.cuda.synchronize()
    k2, v2 = cache.k_cache.clone(), cache.v_cache.clone()
    cache.k_cache.copy_(kc0)
    cache.v_cache.copy_(vc0)
    o1 = torch.empty_like(o2)
    pkv.append(kn, vn, slots_f, cache.k_cache, cache.v_cache, cache.desc)
    pkv.decode(q, cache.k_cache, cache.v_cache, tab, lens, b.shape.scale, o1, cache.desc, mx,
               workspace=ws)
    torch.cuda.synchronize()
    assert torch.equal(o1, o2)
    assert torch.equal(k2.view(torch.uint8), cache.k_cache.view(torch.uint8))
    assert torch.equal(v2.view(torch.uint8), cache.v_cache.view(torch.uint8))
    assert torch.count_nonzero(o2[2]) == 0
    keep = [0, 1, 3]
    st = b.seq_start()
    ref = oracle.decode(b.q[keep], np.concatenate([b.k[st[i]:st[i + 1]] for i in keep]),
                        np.concatenate([b.v[st[i]:st[i + 1]] for i in keep]), b.lens[keep],
                        b.shape.scale)
    assert max_err(o2[keep], ref) <= TOL["bf16"]
