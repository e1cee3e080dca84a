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
from harness import TOL, decode_state, max_err, run_decode, sample_pairs, say

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
    b = synth.cfg2(B=6)
    cache, q, tab, lens, mx = decode_state(b)
    base = run_decode(cache, q, tab, lens, mx, b.shape.scale, partition_tokens=4096)
    for pt in (64, 256, 0):
        o = run_decode(cache, q, tab, lens, mx, b.shape.scale, partition_tokens=pt)
        assert float((o - base).abs().max()) <= 1e-6


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
