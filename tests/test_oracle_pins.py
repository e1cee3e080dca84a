"""Pins of the fp64 oracle to things other than itself (CPU only).

Each test names what fixes the expected value: a closed form, a special case,
an invariant, brute force at 50 digits on tiny inputs, or the worked example
printed on the "LLM Inference: KV Cache, Batching & Scheduling" page.
"""
import json
import math
import os

import mpmath
import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rand(seed, shape, dtype):
    return synth.normal(np.random.default_rng(seed), shape, dtype)


def _as_f64(a):
    a = np.asarray(a)
    return synth.bf16_to_f32(a).astype(np.float64) if a.dtype == np.uint16 else a.astype(np.float64)


# --------------------------------------------------------------------------
# Brute force in 50-digit arithmetic on tiny inputs.

def _mp_attend(q, K, V, scale):
    mpmath.mp.dps = 50
    s = [mpmath.mpf(scale) * mpmath.fsum(mpmath.mpf(float(a)) * mpmath.mpf(float(b))
                                         for a, b in zip(q, k)) for k in K]
    m = max(s)
    e = [mpmath.e ** (x - m) for x in s]
    z = mpmath.fsum(e)
    return [mpmath.fsum(e[j] / z * mpmath.mpf(float(V[j][d])) for j in range(len(K)))
            for d in range(len(V[0]))]


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_decode_matches_mpmath_bruteforce(dtype):
    B, Hq, Hkv, D = 2, 4, 2, 8
    lens = np.array([5, 12])
    q = _rand(11, (B, Hq, D), dtype)
    k = _rand(12, (int(lens.sum()), Hkv, D), dtype)
    v = _rand(13, (int(lens.sum()), Hkv, D), dtype)
    scale = 0.37
    out = oracle.decode(q, k, v, lens, scale)
    qf, kf, vf = _as_f64(q), _as_f64(k), _as_f64(v)
    st = np.concatenate([[0], np.cumsum(lens)])
    G = Hq // Hkv
    for b in range(B):
        for h in range(Hq):
            g = h // G
            ref = _mp_attend(qf[b, h], kf[st[b]:st[b + 1], g], vf[st[b]:st[b + 1], g], scale)
            assert np.max(np.abs(out[b, h] - np.array([float(x) for x in ref]))) <= 1e-13


def test_integer_valued_inputs_match_bruteforce():
    # Integer-valued q/K/V make every logit exact in both precisions.
    g = np.random.default_rng(5)
    q = g.integers(-3, 4, size=(1, 2, 4)).astype(np.float32)
    k = g.integers(-3, 4, size=(7, 1, 4)).astype(np.float32)
    v = g.integers(-5, 6, size=(7, 1, 4)).astype(np.float32)
    out = oracle.decode(q, k, v, [7], 0.25)
    for h in range(2):
        ref = _mp_attend(q[0, h], k[:, 0], v[:, 0], 0.25)
        assert np.max(np.abs(out[0, h] - np.array([float(x) for x in ref]))) <= 1e-13


# --------------------------------------------------------------------------
# Closed forms and special cases.

def test_weights_sum_to_one():
    lens = np.array([1, 3, 40, 257])
    q = _rand(1, (4, 8, 16), "bf16")
    k = _rand(2, (int(lens.sum()), 2, 16), "bf16")
    v = _rand(3, (int(lens.sum()), 2, 16), "bf16")
    for b in range(4):
        for h in (0, 5):
            w, _ = oracle.decode_weights(q, k, v, lens, 0.25, b, h)
            assert len(w) == lens[b]
            assert abs(w.sum() - 1.0) <= 1e-12
            assert np.all(w > 0)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_length_one_returns_v_exactly(dtype):
    q = _rand(21, (3, 4, 32), dtype)
    k = _rand(22, (3, 2, 32), dtype)
    v = _rand(23, (3, 2, 32), dtype)
    out = oracle.decode(q, k, v, [1, 1, 1], 3.0)
    vf = _as_f64(v)
    for b in range(3):
        for h in range(4):
            assert np.array_equal(out[b, h], vf[b, h // 2])


def test_bf16_upcast_known_patterns():
    # 0x3F80 = 1.0, 0xC000 = -2.0, 0x3E80 = 0.25, 0x4049 = 3.140625
    v = np.array([[[0x3F80, 0xC000, 0x3E80, 0x4049]]], dtype=np.uint16)
    q = np.zeros((1, 1, 4), dtype=np.uint16)
    out = oracle.decode(q, v.copy(), v, [1], 1.0)
    assert out[0, 0].tolist() == [1.0, -2.0, 0.25, 3.140625]


@pytest.mark.parametrize("which", ["q_zero", "scale_zero"])
def test_uniform_logits_give_mean_of_v(which):
    L = 37
    q = _rand(31, (1, 4, 16), "f32")
    if which == "q_zero":
        q[:] = 0
    k = _rand(32, (L, 1, 16), "f32")
    v = _rand(33, (L, 1, 16), "f32")
    scale = 0.0 if which == "scale_zero" else 0.5
    out = oracle.decode(q, k, v, [L], scale)
    mean = v[:, 0].astype(np.float64).mean(axis=0)
    for h in range(4):
        assert np.max(np.abs(out[0, h] - mean)) <= 1e-14


def test_equal_keys_give_mean_of_v():
    L = 19
    q = _rand(41, (1, 2, 8), "f32")
    k = np.repeat(_rand(42, (1, 1, 8), "f32"), L, axis=0)
    v = _rand(43, (L, 1, 8), "f32")
    out = oracle.decode(q, k, v, [L], 0.7)
    assert np.max(np.abs(out[0] - v[:, 0].astype(np.float64).mean(axis=0))) <= 1e-14


def test_constant_values_return_constant():
    L = 50
    q = _rand(51, (1, 3, 8), "f32")
    k = _rand(52, (L, 1, 8), "f32")
    v = np.full((L, 1, 8), -1.75, dtype=np.float32)
    out = oracle.decode(q, k, v, [L], 0.3)
    assert np.max(np.abs(out + 1.75)) <= 1e-14


def test_two_keys_logit_gap_ln3():
    # scale*q.k1 - scale*q.k0 = ln 3  =>  weights 1/4 and 3/4, the larger on key 1.
    q = np.zeros((1, 1, 4), dtype=np.float32)
    q[0, 0, 2] = 1.0
    k = np.zeros((2, 1, 4), dtype=np.float32)
    k[1, 0, 2] = 2.0
    k[0, 0, 0] = 9.0       # in a dimension q does not read
    v = np.zeros((2, 1, 4), dtype=np.float32)
    v[0, 0] = [4.0, 0.0, 8.0, -4.0]
    v[1, 0] = [0.0, 8.0, 4.0, 12.0]
    scale = math.log(3.0) / 2.0
    w, row = oracle.decode_weights(q, k, v, [2], scale, 0, 0)
    assert abs(w[0] - 0.25) <= 1e-15 and abs(w[1] - 0.75) <= 1e-15
    assert np.max(np.abs(row - np.array([1.0, 6.0, 5.0, 8.0]))) <= 1e-14


def test_dominant_logit_selects_its_value_row():
    L = 16
    g = np.random.default_rng(61)
    k = g.standard_normal((L, 1, 8)).astype(np.float32) * 0.01
    k[9, 0, :] = 1.0
    q = np.ones((1, 1, 8), dtype=np.float32)
    v = _rand(62, (L, 1, 8), "f32")
    out = oracle.decode(q, k, v, [L], 200.0)
    assert np.max(np.abs(out[0, 0] - v[9, 0])) <= 1e-12


def test_gqa_head_map_contiguous_groups():
    # Hq = 8, Hkv = 2: heads 0..3 read KV head 0, heads 4..7 read KV head 1.
    L = 6
    q = _rand(71, (1, 8, 4), "f32")
    k = _rand(72, (L, 2, 4), "f32")
    v = np.zeros((L, 2, 4), dtype=np.float32)
    v[:, 0, :] = 3.0
    v[:, 1, :] = -5.0
    out = oracle.decode(q, k, v, [L], 1.0)
    assert np.allclose(out[0, :4], 3.0, atol=1e-14, rtol=0)
    assert np.allclose(out[0, 4:], -5.0, atol=1e-14, rtol=0)


def test_empty_context_gives_zeros():
    q = _rand(81, (2, 2, 8), "f32")
    k = _rand(82, (3, 1, 8), "f32")
    out = oracle.decode(q, k, k, [0, 3], 1.0)
    assert np.array_equal(out[0], np.zeros((2, 8)))
    assert np.all(np.isfinite(out[1]))


def test_pairs_subset_matches_full():
    lens = np.array([9, 33, 2])
    q = _rand(91, (3, 4, 16), "bf16")
    k = _rand(92, (int(lens.sum()), 4, 16), "bf16")
    v = _rand(93, (int(lens.sum()), 4, 16), "bf16")
    full = oracle.decode(q, k, v, lens, 0.25)
    pairs = [(1, 3), (2, 0), (0, 2)]
    part = oracle.decode(q, k, v, lens, 0.25, pairs=pairs)
    for b, h in pairs:
        assert np.array_equal(part[b, h], full[b, h])
    assert np.isnan(part[1, 0]).all()


# --------------------------------------------------------------------------
# Chunked prefill: causal boundary and chunk-size independence.

def test_prefill_inclusive_diagonal_and_no_future_leak():
    # One sequence, 3 prior tokens, a 4-token chunk.  Key p0+i has a large
    # logit for query row i; key p0+i+1 (the future) an even larger one.
    p0, C, D = 3, 4, 4
    L = p0 + C
    q = np.zeros((C, 1, D), dtype=np.float32)
    k = np.zeros((L, 1, D), dtype=np.float32)
    for i in range(C):
        q[i, 0, i] = 1.0
        k[p0 + i, 0, i] = 1.0             # row i's own (diagonal) key
        if i + 1 < C:
            k[p0 + i + 1, 0, i] = 2.0     # the next, future key: must stay masked
    v = np.arange(L * D, dtype=np.float32).reshape(L, 1, D)
    out = oracle.prefill(q, [0, C], k, v, [L], 100.0)
    for i in range(C):
        assert np.max(np.abs(out[i, 0] - v[p0 + i, 0])) <= 1e-12


def test_prefill_row_equals_decode_at_that_length():
    prior, C = 11, 6
    pre = synth.custom_prefill(301, [prior], [C], Hq=4, Hkv=2, D=16, block_size=16)
    out = oracle.prefill(pre.q, pre.query_start, pre.k, pre.v, pre.lens, pre.shape.scale)
    for i in range(C):
        L = prior + i + 1
        dq = pre.q[i:i + 1]
        dec = oracle.decode(dq, pre.k[:L], pre.v[:L], [L], pre.shape.scale)
        assert np.array_equal(dec[0], out[i])


def test_prefill_chunk_size_independence():
    # The same 24-token prompt over 5 prior tokens, prefilled as one chunk,
    # as 3 chunks of 8 and as 24 chunks of 1: every query row is identical.
    prior, n = 5, 24
    full = synth.custom_prefill(302, [prior], [n], Hq=4, Hkv=1, D=8, block_size=16)
    ref = oracle.prefill(full.q, full.query_start, full.k, full.v, full.lens, full.shape.scale)
    for csz in (8, 1):
        rows = []
        for c0 in range(0, n, csz):
            L = prior + c0 + csz
            o = oracle.prefill(full.q[c0:c0 + csz], [0, csz], full.k[:L], full.v[:L], [L],
                               full.shape.scale)
            rows.append(o)
        assert np.array_equal(np.concatenate(rows), ref)


def test_prefill_zero_prior_first_row_is_v0():
    pre = synth.custom_prefill(303, [0, 4], [5, 3], Hq=2, Hkv=1, D=8, block_size=16)
    out = oracle.prefill(pre.q, pre.query_start, pre.k, pre.v, pre.lens, pre.shape.scale)
    v0 = synth.bf16_to_f32(pre.v[0, 0]).astype(np.float64)
    assert np.array_equal(out[0, 0], v0) and np.array_equal(out[0, 1], v0)


# Several sequences in one call: priors 0, 7, 3, 12 and 2, chunks 5, 1, 0, 4
# and 3 (a zero prior, a one-token chunk, an empty chunk between two
# non-empty ones).  Every chunk row must attend exactly its own sequence's
# keys 0 .. p0 + i ("Chunked prefill": splitting the prompt into chunks, and
# batching chunks of several prompts in one step, leaves each row's result as
# the unsplit prompt's).
_MS_PRIOR, _MS_CHUNK = [0, 7, 3, 12, 2], [5, 1, 0, 4, 3]


def _multi_seq_prefill(dtype):
    return synth.custom_prefill(304, _MS_PRIOR, _MS_CHUNK, Hq=4, Hkv=2, D=8, block_size=16,
                                dtype=dtype)


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_prefill_multi_sequence_rows_match_mpmath(dtype):
    # Brute force at 50 digits for every row of every sequence, with the
    # sequence, the row's position in its chunk and the key range worked out
    # here from the chunk lengths (not from the oracle's row lookup).
    pre = _multi_seq_prefill(dtype)
    out = oracle.prefill(pre.q, pre.query_start, pre.k, pre.v, pre.lens, pre.shape.scale)
    qf, kf, vf = _as_f64(pre.q), _as_f64(pre.k), _as_f64(pre.v)
    G = pre.shape.Hq // pre.shape.Hkv
    r, kv0 = 0, 0
    for p0, C in zip(_MS_PRIOR, _MS_CHUNK):
        for i in range(C):
            keys = slice(kv0, kv0 + p0 + i + 1)
            for h in range(pre.shape.Hq):
                ref = _mp_attend(qf[r, h], kf[keys, h // G], vf[keys, h // G], pre.shape.scale)
                assert np.max(np.abs(out[r, h] - np.array([float(x) for x in ref]))) <= 1e-13, \
                    (r, h)
            r += 1
        kv0 += p0 + C
    assert r == out.shape[0]


def test_prefill_multi_sequence_rows_equal_single_sequence_decode():
    # Row i of sequence b equals a one-sequence decode over that sequence's
    # first p0 + i + 1 rows (the sequence's own K/V cut out here by hand).
    pre = _multi_seq_prefill("bf16")
    out = oracle.prefill(pre.q, pre.query_start, pre.k, pre.v, pre.lens, pre.shape.scale)
    r, kv0 = 0, 0
    for p0, C in zip(_MS_PRIOR, _MS_CHUNK):
        for i in range(C):
            L = p0 + i + 1
            dec = oracle.decode(pre.q[r:r + 1], pre.k[kv0:kv0 + L], pre.v[kv0:kv0 + L], [L],
                                pre.shape.scale)
            assert np.array_equal(dec[0], out[r]), r
            r += 1
        kv0 += p0 + C


def test_prefill_multi_sequence_rows_subset_matches_full():
    # The row-subset path: each (row, head) pair computed alone equals the
    # full call, for the first and last row of every non-empty chunk.
    pre = _multi_seq_prefill("bf16")
    full = oracle.prefill(pre.q, pre.query_start, pre.k, pre.v, pre.lens, pre.shape.scale)
    qs = pre.query_start
    rows = sorted({int(x) for b in range(len(_MS_CHUNK)) if qs[b + 1] > qs[b]
                   for x in (qs[b], qs[b + 1] - 1)})
    pairs = np.array([(r, h) for r in rows for h in range(pre.shape.Hq)], dtype=np.int32)
    part = oracle.prefill(pre.q, pre.query_start, pre.k, pre.v, pre.lens, pre.shape.scale,
                          rows=pairs)
    for r, h in pairs:
        assert np.array_equal(part[r, h], full[r, h])


# --------------------------------------------------------------------------
# Append: a tiny cache image written out by hand, plus invariants.

def test_append_tiny_image_by_hand():
    # 2 blocks x 1 KV head x block 4 x D 4, float32 (E = 4 dims per chunk,
    # so a K tile is row-major and a V tile is its transpose); slots
    # [5, -1, 0]: slot 5 -> block 1, offset 1; slot 0 -> block 0, offset 0.
    k = np.array([[[1, 2, 3, 4]], [[5, 6, 7, 8]], [[9, 10, 11, 12]]], dtype=np.float32)
    v = -k
    kc = np.full((2, 1, 4, 4), 99.0, dtype=np.float32)
    vc = np.full((2, 1, 4, 4), 99.0, dtype=np.float32)
    oracle.append(k, v, [5, -1, 0], kc, vc, 4)
    ek = np.full(32, 99.0, dtype=np.float32)
    ek[16 + 4:16 + 8] = [1, 2, 3, 4]          # block 1, token 1: K row 1 of the tile
    ek[0:4] = [9, 10, 11, 12]                 # block 0, token 0: K row 0
    ev = np.full(32, 99.0, dtype=np.float32)
    ev[[16 + 1, 16 + 5, 16 + 9, 16 + 13]] = [-1, -2, -3, -4]   # block 1: V column 1
    ev[[0, 4, 8, 12]] = [-9, -10, -11, -12]                     # block 0: V column 0
    assert np.array_equal(kc.reshape(-1), ek)
    assert np.array_equal(vc.reshape(-1), ev)


def test_append_chunked_positions_by_hand():
    # bf16, block 8, D 16 (E = 8): token 5 of block 0, dim 10 lands at
    # K index ((10 // 8) * 8 + 5) * 8 + 2 = 106 and V index
    # ((5 // 4) * 16 + 10) * 4 + 1 = 105 (worked by hand).
    k = np.zeros((1, 1, 16), dtype=np.uint16)
    v = np.zeros((1, 1, 16), dtype=np.uint16)
    k[0, 0, 10] = 0x1234
    v[0, 0, 10] = 0x5678
    kc = np.zeros((1, 1, 8, 16), dtype=np.uint16)
    vc = np.zeros_like(kc)
    oracle.append(k, v, [5], kc, vc, 8)
    assert np.flatnonzero(kc.reshape(-1)).tolist() == [106]
    assert np.flatnonzero(vc.reshape(-1)).tolist() == [105]
    assert kc.reshape(-1)[106] == 0x1234 and vc.reshape(-1)[105] == 0x5678
    assert oracle.tile_index(5, 10, 8, 16, 2) == (106, 105)
    # f32, block 16, D 8 (E = 4): token 9, dim 6 -> K (1 * 16 + 9) * 4 + 2 = 102,
    # V (2 * 8 + 6) * 4 + 1 = 89.
    assert oracle.tile_index(9, 6, 16, 8, 4) == (102, 89)


def _row(cache_tile: np.ndarray, t: int, bs: int, D: int, which: int) -> np.ndarray:
    flat = cache_tile.reshape(-1)
    es = cache_tile.dtype.itemsize
    return np.array([flat[oracle.tile_index(t, d, bs, D, es)[which]] for d in range(D)],
                    dtype=cache_tile.dtype)


def test_append_bits_preserved_and_nothing_else_touched():
    g = np.random.default_rng(7)
    nb, H, bs, D, T = 10, 2, 16, 8, 40
    k = g.integers(0, 2**16, size=(T, H, D), dtype=np.uint16)
    v = g.integers(0, 2**16, size=(T, H, D), dtype=np.uint16)
    slots = g.permutation(nb * bs)[:T].astype(np.int32)
    slots[::7] = -1
    kc = np.full((nb, H, bs, D), synth.POISON_BF16, dtype=np.uint16)
    vc = kc.copy()
    oracle.append(k, v, slots, kc, vc, bs)
    written = int((slots >= 0).sum()) * H * D
    assert int((kc != synth.POISON_BF16).sum()) <= written
    # Logical read-back: every appended row is found where its slot says.
    for t, s in enumerate(slots):
        if s >= 0:
            for h in range(H):
                assert np.array_equal(_row(kc[s // bs, h], s % bs, bs, D, 0), k[t, h])
                assert np.array_equal(_row(vc[s // bs, h], s % bs, bs, D, 1), v[t, h])
    # Untouched slots keep the poison in every head.
    used = set(int(s) for s in slots if s >= 0)
    for s in range(nb * bs):
        if s not in used:
            for h in range(H):
                assert np.all(_row(kc[s // bs, h], s % bs, bs, D, 0) == synth.POISON_BF16)
                assert np.all(_row(vc[s // bs, h], s % bs, bs, D, 1) == synth.POISON_BF16)


def test_append_rejects_out_of_range_slot():
    k = np.zeros((1, 1, 4), dtype=np.float32)
    kc = np.zeros((2, 1, 4, 4), dtype=np.float32)
    with pytest.raises(ValueError):
        oracle.append(k, k, [8], kc, kc.copy(), 4)


# --------------------------------------------------------------------------
# The page's worked sizing example.

# --------------------------------------------------------------------------
# Block copy: a hand-written image, logical read-back through the slot rule,
# and the skip rule.

def test_copy_blocks_tiny_image_by_hand():
    # 3 blocks x 1 KV head x block 2 x D 2, float32; copy block 2 -> block 0.
    kc = np.arange(12, dtype=np.float32).reshape(3, 1, 2, 2)
    vc = -kc
    oracle.copy_blocks(kc, vc, kc, vc, [2], [0])
    exp = np.array([8, 9, 10, 11, 4, 5, 6, 7, 8, 9, 10, 11], dtype=np.float32).reshape(3, 1, 2, 2)
    assert np.array_equal(kc, exp) and np.array_equal(vc, -exp)


def test_copy_blocks_preserves_logical_rows_through_append():
    # A sequence written by append through block list [a, b]; after copying
    # a -> c and b -> d, reading the sequence through [c, d] gives the rows
    # that were appended, in order, for every head.
    g = np.random.default_rng(11)
    nb, H, bs, D, T = 8, 3, 4, 16, 7
    k = g.integers(0, 2**16, size=(T, H, D), dtype=np.uint16)
    v = g.integers(0, 2**16, size=(T, H, D), dtype=np.uint16)
    blocks = [5, 2]
    slots = [blocks[t // bs] * bs + t % bs for t in range(T)]
    kc = np.zeros((nb, H, bs, D), dtype=np.uint16)
    vc = np.zeros_like(kc)
    oracle.append(k, v, slots, kc, vc, bs)
    dk, dv = np.zeros_like(kc), np.zeros_like(vc)
    oracle.copy_blocks(kc, vc, dk, dv, blocks, [0, 7])
    new = [0, 7]
    for t in range(T):
        for h in range(H):
            assert np.array_equal(_row(dk[new[t // bs], h], t % bs, bs, D, 0), k[t, h])
            assert np.array_equal(_row(dv[new[t // bs], h], t % bs, bs, D, 1), v[t, h])
    untouched = [b for b in range(nb) if b not in new]
    assert not dk[untouched].any() and not dv[untouched].any()


def test_copy_blocks_skips_out_of_range_pairs():
    kc = np.arange(2 * 2 * 2 * 4, dtype=np.float32).reshape(2, 2, 2, 4)
    vc = kc + 100
    dk, dv = np.full_like(kc, -1), np.full_like(vc, -1)
    oracle.copy_blocks(kc, vc, dk, dv, [-1, 2, 0, 1], [0, 1, 2, 1])
    assert np.all(dk[0] == -1)                      # src -1: skipped
    assert np.array_equal(dk[1], kc[1]) and np.array_equal(dv[1], vc[1])   # only (1 -> 1)


# --------------------------------------------------------------------------
# Prefix cache: reusable tokens, worked by hand.

@pytest.mark.parametrize("prompt,cached,bs,expect", [
    ([1, 2, 3, 4, 5, 6, 7, 8, 9], [[1, 2, 3, 4, 5, 6, 7, 8]], 4, 8),
    ([1, 2, 3, 4, 5, 6, 7, 8], [[1, 2, 3, 4, 5, 6, 7, 8]], 4, 4),    # one token left to compute
    ([1, 2, 3, 4, 5, 6, 7, 0, 9], [[1, 2, 3, 4, 5, 6, 7, 8]], 4, 4),  # second block differs
    ([0, 2, 3, 4, 5, 6, 7, 8, 9], [[1, 2, 3, 4, 5, 6, 7, 8]], 4, 0),  # first token differs
    ([1, 2, 3, 4, 5, 6, 7, 8, 9], [[1, 2, 3], [1, 2, 3, 4, 5]], 4, 4),
    ([], [[1, 2]], 2, 0),
    ([7], [[7]], 1, 0),
    ([7, 8], [[7, 8, 9]], 1, 1),
])
def test_reusable_prefix_tokens_by_hand(prompt, cached, bs, expect):
    assert oracle.reusable_prefix_tokens(prompt, cached, bs) == expect


def test_kv_sizing_worked_example():
    with open(os.path.join(GOLDEN, "kv_sizing.json")) as f:
        ex = json.load(f)
    per_tok_layer = oracle.kv_bytes_per_layer(1, ex["kv_heads"], ex["head_dim"], ex["dtype_bytes"])
    assert per_tok_layer == ex["per_layer_bytes_per_token"]
    assert oracle.kv_bytes_per_layer(1000, 8, 128, 2) == 4096 * 1000
    per_tok = per_tok_layer * ex["layers"]
    assert per_tok == ex["per_token_all_layers_bytes"]
    req = oracle.kv_bytes_per_layer(ex["request_tokens"], 8, 128, 2) * ex["layers"]
    assert req == 1342177280
    # The printed "1.28 GB" is this byte count in units of 1000 * 2^20 bytes.
    assert round(req / (1000 * 2**20), 2) == ex["request_printed_gb"]
    # "About 30" concurrent requests: the 38 GB left over divided by 1.28.
    assert round(ex["hbm_left_gb"] / ex["request_printed_gb"]) == ex["concurrent_requests_printed"]
    assert ex["hbm_total_gb"] - ex["weights_gb"] == ex["hbm_left_gb"]
