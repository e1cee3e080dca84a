"""Causal chunked prefill on the MFMA path against the fp64 oracle ("LLM
Inference: KV Cache, Batching & Scheduling", section "Chunked prefill": a
chunk of the prompt attends every earlier key and itself, and splitting the
prompt into chunks does not change the result).

Bar: max abs error 2e-3 for bf16 inputs on fp32 output; bitwise equality for
the placement and poison invariants.
"""
import numpy as np
import pytest
import torch

import oracle
import paged_kv_cache_indirected_amd as pkv
import synth
from harness import (TOL, decode_state, max_err, prefill_state, run_decode, run_prefill,
                     sample_rows, say)

pytestmark = pytest.mark.gpu


def _check(batch, rows=None, label=""):
    C = int(batch.chunk.max())
    say(f"[prefill] {label} S={len(batch.chunk)} prior={batch.prior.tolist()} "
        f"chunk={batch.chunk.tolist()} G={batch.shape.Hq // batch.shape.Hkv} "
        f"D={batch.shape.D} bs={batch.shape.block_size}")
    st = prefill_state(batch)
    out = run_prefill(*st, batch.shape.scale, C)
    ref = oracle.prefill(batch.q, batch.query_start, batch.k, batch.v, batch.lens,
                         batch.shape.scale, rows=rows)
    o = out.float().cpu().numpy().astype(np.float64)
    if rows is None:
        err = float(np.max(np.abs(o - ref))) if o.size else 0.0
    else:
        err = max(float(np.max(np.abs(o[t, h] - ref[t, h]))) for t, h in rows)
    say(f"  max abs err {err:.3e}")
    assert np.isfinite(err) and err <= TOL["bf16"], err
    return out


def test_cfg5_prefill_sampled():
    pre, _ = synth.cfg5()
    T = int(pre.chunk.sum())
    _check(pre, rows=sample_rows(T, pre.shape.Hq, 1024, 51), label="cfg5")


def test_cfg5_prefill_first_and_last_rows_full():
    # Every head of the first and last token of each chunk: the shortest and
    # the longest rows, the diagonal tile included.
    pre, _ = synth.cfg5()
    qs = pre.query_start
    rows = [(int(t), h) for b in range(len(pre.chunk))
            for t in (qs[b], qs[b] + 1, qs[b + 1] - 1) for h in range(pre.shape.Hq)]
    _check(pre, rows=np.array(rows, dtype=np.int32), label="cfg5-edges")


@pytest.mark.parametrize("D", [64, 128])
@pytest.mark.parametrize("bs", [16, 32])
@pytest.mark.parametrize("G", [1, 2, 4, 8])
def test_shape_sweep_ragged(D, bs, G):
    # Priors at 0, inside a block, on a block boundary; chunks of 1, ragged
    # against the 128-row tile and the 64-key tile.
    b = synth.custom_prefill(300 + G + D + bs, prior=[0, 5, 64, 200], chunk=[37, 1, 130, 77],
                             Hq=2 * G, Hkv=2, D=D, block_size=bs)
    _check(b, label="sweep")


@pytest.mark.parametrize("split", [False, True])
def test_empty_chunk_and_max_query_len_above_every_chunk(split):
    # A sequence with no chunk rows between two that have some, and a
    # max_query_len (and so a grid and a split workspace) larger than any
    # chunk: the rows that exist match the oracle, nothing else is written.
    b = synth.custom_prefill(318, prior=[10, 3000, 0], chunk=[20, 0, 5], Hq=16, Hkv=2, D=128,
                             block_size=16)
    say(f"[prefill] empty chunk, max_query_len 200, split={split}")
    cache, q, qs, tab, lens, mx = prefill_state(b)
    T, Hq, D = q.shape
    out = torch.full((T + 3, Hq, D), 7.0, dtype=torch.float32, device=q.device)
    ws = None
    if split:
        n = pkv.prefill_workspace_bytes(3, Hq, 200, cache.desc)
        ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    pkv.prefill_chunk(q, qs, cache.k_cache, cache.v_cache, tab, lens, b.shape.scale, out[:T],
                      cache.desc, 200, mx, workspace=ws)
    torch.cuda.synchronize()
    ref = oracle.prefill(b.q, b.query_start, b.k, b.v, b.lens, b.shape.scale)
    assert max_err(out[:T], ref) <= TOL["bf16"]
    assert torch.all(out[T:] == 7.0)


@pytest.mark.parametrize("split", [False, True])
@pytest.mark.parametrize("bs,prior", [(16, 17000), (32, 33000)])
def test_block_table_longer_than_the_id_ring(split, bs, prior):
    # More than 1024 blocks in a sequence's table: the kernel's LDS ring of
    # block ids is restaged as the loop moves on (more than 2 x 128 key tiles
    # at block 16, 2 x 256 at block 32).
    b = synth.custom_prefill(319, prior=[prior, 30], chunk=[40, 9], Hq=16, Hkv=2, D=128,
                             block_size=bs)
    say(f"[prefill] long table ({int(b.lens.max()) // bs + 1} blocks), bs={bs}, split={split}")
    cache, q, qs, tab, lens, mx = prefill_state(b)
    assert tab.shape[1] > 1024
    out = run_prefill(cache, q, qs, tab, lens, mx, b.shape.scale, 40, split=split)
    ref = oracle.prefill(b.q, b.query_start, b.k, b.v, b.lens, b.shape.scale)
    assert max_err(out, ref) <= TOL["bf16"]


def test_first_chunk_of_a_prompt_p0_zero():
    b = synth.custom_prefill(310, prior=[0, 0], chunk=[512, 3], Hq=64, Hkv=8, D=128,
                             block_size=16)
    _check(b, label="p0=0")


def test_prefill_row_equals_decode_at_that_length():
    b = synth.custom_prefill(311, prior=[100], chunk=[40], Hq=16, Hkv=2, D=128, block_size=16)
    st = prefill_state(b)
    out = run_prefill(*st, b.shape.scale, 40).cpu().numpy()
    for i in (0, 17, 39):
        L = 100 + i + 1
        dec = synth.DecodeBatch(0, "row", b.shape, np.array([L]), b.q[i:i + 1], b.k[:L], b.v[:L],
                                pool_blocks=64, pool_seed=5)
        o_dec = run_decode(*decode_state(dec), b.shape.scale).cpu().numpy()
        assert np.max(np.abs(out[i] - o_dec[0])) <= 2 * TOL["bf16"]


def test_chunk_split_independence():
    # One 256-token chunk vs the same prompt prefilled as 4 chunks of 64.
    whole = synth.custom_prefill(312, prior=[300], chunk=[256], Hq=16, Hkv=2, D=128,
                                 block_size=16)
    o_whole = run_prefill(*prefill_state(whole), whole.shape.scale, 256).cpu().numpy()
    parts = []
    for c in range(4):
        P = 300 + 64 * c
        L = P + 64
        pb = synth.PrefillBatch(whole.shape, np.array([P]), np.array([64]),
                                whole.q[64 * c:64 * (c + 1)], whole.k[:L], whole.v[:L],
                                pool_blocks=64, pool_seed=9 + c)
        parts.append(run_prefill(*prefill_state(pb), whole.shape.scale, 64).cpu().numpy())
    o_parts = np.concatenate(parts)
    assert np.max(np.abs(o_whole - o_parts)) <= 2 * TOL["bf16"]
    ref = oracle.prefill(whole.q, whole.query_start, whole.k, whole.v, whole.lens,
                         whole.shape.scale)
    assert np.max(np.abs(o_parts - ref)) <= TOL["bf16"]


def test_placement_and_poison_bitwise():
    b = synth.custom_prefill(313, prior=[33, 0], chunk=[70, 20], Hq=16, Hkv=2, D=128,
                             block_size=16)
    outs = [run_prefill(*prefill_state(b, pool_seed=s, poison=p), b.shape.scale, 70)
            for s, p in ((None, None), (0, None), (77, 0x0000), (5, 0x7F7F))]
    assert torch.isfinite(outs[0]).all()
    for o in outs[1:]:
        assert torch.equal(outs[0], o)


def test_bf16_output():
    b = synth.custom_prefill(314, prior=[128], chunk=[64], Hq=64, Hkv=8, D=128, block_size=16)
    out = run_prefill(*prefill_state(b), b.shape.scale, 64, out_dtype=torch.bfloat16)
    ref = oracle.prefill(b.q, b.query_start, b.k, b.v, b.lens, b.shape.scale)
    o = out.float().cpu().numpy().astype(np.float64)
    half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 8)
    assert np.all(np.abs(o - ref) <= 2e-3 + half_ulp)


@pytest.mark.parametrize("case", [
    # (prior, chunk, Hq, Hkv, D, bs): few workgroups over long contexts, so
    # the library splits the keys; the short sequence beside the long one has
    # fewer key tiles than splits (empty splits).
    ([3000, 0], [64, 16], 16, 2, 128, 16),
    ([4000], [200], 64, 8, 128, 16),
    ([2500, 1200, 7], [33, 128, 5], 8, 8, 64, 32),
])
def test_key_splits_match_single_pass_and_oracle(case):
    prior, chunk, Hq, Hkv, D, bs = case
    b = synth.custom_prefill(316 + len(prior), prior=prior, chunk=chunk, Hq=Hq, Hkv=Hkv, D=D,
                             block_size=bs)
    C = int(b.chunk.max())
    ws = pkv.prefill_workspace_bytes(len(chunk), Hq, C, pkv.CacheDesc(
        b.pool_blocks, Hkv, bs, D, pkv.BF16))
    assert ws > 0, "expected a key-split workspace for this shape"
    st = prefill_state(b)
    o_split = run_prefill(*st, b.shape.scale, C, split=True)
    o_one = run_prefill(*st, b.shape.scale, C, split=False)
    say(f"[prefill] key splits prior={prior} chunk={chunk}: split vs single "
        f"{(o_split - o_one).abs().max().item():.3e}")
    # The merge is an exact rearrangement of the softmax sums: the two differ
    # by fp32 rounding only.
    assert torch.allclose(o_split, o_one, rtol=0, atol=1e-5)
    ref = oracle.prefill(b.q, b.query_start, b.k, b.v, b.lens, b.shape.scale)
    err = float(np.max(np.abs(o_split.cpu().numpy().astype(np.float64) - ref)))
    assert np.isfinite(err) and err <= TOL["bf16"], err
    # A workspace shorter than asked for: the library splits less (or not
    # at all) and the result is the same up to fp32 rounding.
    cache, q, qs, tables, lens, mx = st
    for frac in (2, 5):
        short = torch.empty(ws // frac, dtype=torch.uint8, device="cuda")
        o_short = torch.empty_like(o_one)
        pkv.prefill_chunk(q, qs, cache.k_cache, cache.v_cache, tables, lens, b.shape.scale,
                          o_short, cache.desc, C, mx, workspace=short)
        torch.cuda.synchronize()
        assert torch.allclose(o_short, o_one, rtol=0, atol=1e-5), frac
    o_bf = run_prefill(*st, b.shape.scale, C, out_dtype=torch.bfloat16, split=True)
    half_ulp = 2.0 ** (np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 8)
    assert np.all(np.abs(o_bf.float().cpu().numpy().astype(np.float64) - ref) <= 2e-3 + half_ulp)


def test_repeat_is_bitwise_deterministic():
    b = synth.custom_prefill(315, prior=[500], chunk=[128], Hq=64, Hkv=8, D=128, block_size=16)
    st = prefill_state(b)
    o1 = run_prefill(*st, b.shape.scale, 128)
    o2 = run_prefill(*st, b.shape.scale, 128)
    assert torch.equal(o1, o2)


@pytest.mark.parametrize("split", [False, True])
def test_out_of_range_block_id_reads_zeros(split):
    # A block id outside the pool inside the context (a precondition
    # violation) is read as zero keys and values, never from memory: the
    # oracle gets zeros for those rows.
    b = synth.custom_prefill(315, prior=[200, 40], chunk=[48, 32], Hq=16, Hkv=2, D=128,
                             block_size=16)
    cache, q, qs, tables, lens, mx = prefill_state(b)
    bs = b.shape.block_size
    k, v = b.k.copy(), b.v.copy()
    start = np.concatenate([[0], np.cumsum(b.lens)])
    for s, j, bad in ((0, 3, cache.desc.num_blocks + 5), (0, 9, -3), (1, 1, 1 << 30)):
        tables[s, j] = bad
        r0 = start[s] + j * bs
        k[r0:r0 + bs] = 0
        v[r0:r0 + bs] = 0
    C = int(b.chunk.max())
    out = run_prefill(cache, q, qs, tables, lens, mx, b.shape.scale, C, split=split)
    ref = oracle.prefill(b.q, b.query_start, k, v, b.lens, b.shape.scale)
    err = float(np.max(np.abs(out.float().cpu().numpy().astype(np.float64) - ref)))
    say(f"[prefill] out-of-range ids, split={split}: max abs err {err:.3e}")
    assert np.isfinite(err) and err <= TOL["bf16"], err
