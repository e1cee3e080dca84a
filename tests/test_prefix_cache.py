"""Prefix cache, fork and copy-on-write in the host pool (CPU only).

Follows "LLM Inference: KV Cache, Batching & Scheduling", "Prefix caching"
(a shared prefix's KV is computed once; later requests pay only for the
tokens after it) and the "LLM Inference Engineering" summary, section 2
(identical prefixes share pages).  The expected number of reusable tokens
comes from the oracle's definition (longest whole-block common prefix with an
earlier prompt, at least one token left to compute).
"""
import numpy as np
import pytest

import oracle
import paged_kv_cache_indirected_amd as pkv


def _prompt_seq(s, sid, tokens):
    """Admit a prompt through the prefix cache, 'prefill' the rest, register it."""
    reused = s.add_cached(sid, tokens)
    s.append(sid, len(tokens) - reused)
    s.cache(sid, tokens)
    return reused


def test_second_request_reuses_whole_prefix_blocks():
    p = pkv.Pool(64)
    s = pkv.Seqs(p, 4)
    a = list(range(100, 111))                 # 11 tokens: 2 full blocks + 3
    assert _prompt_seq(s, 0, a) == 0
    b = a[:9] + [7, 7, 7]                     # shares 9 tokens -> 2 whole blocks
    assert _prompt_seq(s, 1, b) == 8
    assert s.block_ids(1)[:2] == s.block_ids(0)[:2]
    assert s.block_ids(1)[2] != s.block_ids(0)[2]
    assert p.refcount(s.block_ids(0)[0]) == 2


def test_identical_prompt_leaves_one_token_to_compute():
    p = pkv.Pool(64)
    s = pkv.Seqs(p, 4)
    a = list(range(8))
    _prompt_seq(s, 0, a)
    assert s.add_cached(1, a) == 4            # (8 - 1) // 4 = 1 block
    assert s.length(1) == 4


def test_chain_key_depends_on_whole_prefix():
    # Same second block, different first block: nothing is reused.
    p = pkv.Pool(64)
    s = pkv.Seqs(p, 2)
    _prompt_seq(s, 0, [1, 2, 3, 4, 5])
    assert s.add_cached(1, [9, 9, 3, 4, 5]) == 0


def test_released_cached_blocks_stay_reusable_until_evicted():
    p = pkv.Pool(6)
    s = pkv.Seqs(p, 4)
    a = list(range(12))                       # 3 full blocks
    _prompt_seq(s, 0, a + [99])               # 4 blocks in use (last partial)
    blocks = s.block_ids(0)
    s.release(0)
    assert p.num_cached == 3 and p.num_free == 6
    assert all(p.refcount(b) == 0 for b in blocks)
    # A new request with the same prefix revives the cached blocks.
    assert s.add_cached(1, a + [5]) == 12
    assert s.block_ids(1) == blocks[:3] and p.num_cached == 0
    assert all(p.refcount(b) == 1 for b in blocks[:3])


def test_eviction_takes_free_list_first_then_least_recently_released():
    p = pkv.Pool(4)
    s = pkv.Seqs(p, 2)
    _prompt_seq(s, 0, [1, 2, 3])              # blocks x0 (full, cached), x1 (partial)
    _prompt_seq(s, 1, [5, 6, 7])              # blocks y0 (cached), y1
    x0, y0 = s.block_ids(0)[0], s.block_ids(1)[0]
    s.release(0)                               # x0 -> LRU (older)
    s.release(1)                               # y0 -> LRU (newer)
    assert p.num_cached == 2 and p.num_free == 4
    # Two plain blocks come from the free list; the cache is untouched.
    s.add(2)
    s.append(2, 4)
    assert p.num_cached == 2
    # The next block evicts x0 (least recently released), not y0.
    s.append(2, 1)
    assert x0 in s.block_ids(2) and p.num_cached == 1
    assert s.add_cached(3, [1, 2, 3]) == 0    # x0's entry is gone
    s.release(3)
    assert s.add_cached(4, [5, 6, 7]) == 2    # y0 still cached
    assert s.block_ids(4) == [y0]


def test_exhaustion_with_cache_is_all_or_nothing():
    p = pkv.Pool(3)
    s = pkv.Seqs(p, 2)
    _prompt_seq(s, 0, [1, 2, 3])              # 2 blocks
    s.release(0)
    s.add(1)
    with pytest.raises(pkv.PkvError) as e:
        s.append(1, 8)                        # 4 blocks > 3
    assert e.value.code == pkv.ENOBLOCKS
    assert p.num_cached == 1 and p.num_free == 3 and s.length(1) == 0


def test_cache_rejects_more_tokens_than_written():
    p = pkv.Pool(8)
    s = pkv.Seqs(p, 4)
    s.add(0)
    s.append(0, 5)
    with pytest.raises(pkv.PkvError) as e:
        s.cache(0, list(range(6)))
    assert e.value.code == pkv.EINVAL
    with pytest.raises(pkv.PkvError) as e:
        s.add_cached(0, [1, 2, 3])
    assert e.value.code == pkv.ESTATE


def test_reregistering_a_block_replaces_its_old_entry():
    p = pkv.Pool(8)
    s = pkv.Seqs(p, 2)
    s.add(0)
    s.append(0, 2)
    s.cache(0, [1, 2])
    s.cache(0, [3, 4])                        # the block now holds other tokens
    assert s.add_cached(1, [1, 2, 0]) == 0
    assert s.add_cached(2, [3, 4, 0]) == 2


@pytest.mark.parametrize("seed", [1, 2, 3])
def test_random_workload_matches_reusable_prefix_definition(seed):
    # Prompts drawn from a few shared "system prompts" plus private tails.
    # With a pool large enough that nothing is evicted, every admission
    # reuses exactly what the oracle's definition says.
    g = np.random.default_rng(seed)
    bs = 4
    bases = [list(g.integers(0, 50, size=g.integers(0, 30))) for _ in range(4)]
    p = pkv.Pool(4096)
    s = pkv.Seqs(p, bs)
    earlier = []
    for sid in range(40):
        base = bases[g.integers(0, len(bases))]
        cut = int(g.integers(0, len(base) + 1))
        prompt = [int(t) for t in base[:cut]] + [int(t) for t in g.integers(0, 50, size=g.integers(1, 9))]
        expect = oracle.reusable_prefix_tokens(prompt, earlier, bs)
        assert _prompt_seq(s, sid, prompt) == expect
        earlier.append(prompt)
        if g.random() < 0.3:
            s.release(sid)


# --------------------------------------------------------------------------
# Fork and copy-on-write.

def test_fork_shares_every_block_including_the_partial_one():
    p = pkv.Pool(16)
    s = pkv.Seqs(p, 4)
    s.add(0)
    s.append(0, 6)
    s.fork(1, 0)
    assert s.block_ids(1) == s.block_ids(0) and s.length(1) == 6
    assert all(p.refcount(b) == 2 for b in s.block_ids(0))
    with pytest.raises(pkv.PkvError) as e:
        s.append(1, 1)                        # plain append refuses a shared block
    assert e.value.code == pkv.ESTATE


def test_append_cow_copies_the_shared_partial_block_once():
    p = pkv.Pool(16)
    s = pkv.Seqs(p, 4)
    s.add(0)
    s.append(0, 6)
    old = s.block_ids(0)
    s.fork(1, 0)
    slots, copies = s.append_cow(1, 3)        # 6 -> 9: into the partial block, then a new one
    new = s.block_ids(1)
    assert copies == [(old[1], new[1])] and new[0] == old[0] and new[1] != old[1]
    assert list(slots) == [new[1] * 4 + 2, new[1] * 4 + 3, new[2] * 4 + 0]
    assert p.refcount(old[1]) == 1 and p.refcount(new[1]) == 1 and p.refcount(old[0]) == 2
    # Sequence 0 now holds its last block alone: no copy.
    slots0, copies0 = s.append_cow(0, 1)
    assert copies0 == [] and slots0[0] == old[1] * 4 + 2
    # A full shared block needs no copy either.
    s.fork(2, 0)
    _, copies = s.append_cow(0, 1)            # fills block old[1], now shared again
    assert len(copies) == 1 and copies[0][0] == old[1] and s.length(0) == 8
    _, copies = s.append_cow(2, 1)            # seq 2 is the last holder of old[1]
    assert copies == [] and p.refcount(old[1]) == 1


def test_append_cow_all_or_nothing():
    p = pkv.Pool(2)
    s = pkv.Seqs(p, 4)
    s.add(0)
    s.append(0, 6)                            # both blocks used
    s.fork(1, 0)
    with pytest.raises(pkv.PkvError) as e:
        s.append_cow(1, 1)
    assert e.value.code == pkv.ENOBLOCKS
    assert s.block_ids(1) == s.block_ids(0) and s.length(1) == 6


@pytest.mark.parametrize("order", [[0, 1, 2], [2, 0, 1], [1, 2]])
def test_batch_cow_last_holder_keeps_the_original(order):
    p = pkv.Pool(32)
    s = pkv.Seqs(p, 4)
    s.add(0)
    s.append(0, 5)
    s.fork(1, 0)
    s.fork(2, 0)
    shared = s.block_ids(0)[1]
    free0 = p.num_free
    slots, copies = s.append_batch_cow(order)
    holders = 3
    n_copy = len(order) - (1 if len(order) == holders else 0)
    assert len(copies) == n_copy and p.num_free == free0 - n_copy
    assert all(c[0] == shared for c in copies)
    last = [s.block_ids(i)[1] for i in range(3)]
    assert last.count(shared) == holders - n_copy
    assert p.refcount(shared) == holders - n_copy
    # Every slot is in its sequence's own (now private) last block.
    for i, sid in enumerate(order):
        assert slots[i] == s.block_ids(sid)[1] * 4 + 1
        assert p.refcount(s.block_ids(sid)[1]) == 1


def test_batch_cow_exact_allocation_at_the_limit():
    # Two holders, both in the batch: exactly one fresh block is needed.
    p = pkv.Pool(2)
    s = pkv.Seqs(p, 4)
    s.add(0)
    s.append(0, 3)
    s.fork(1, 0)
    slots, copies = s.append_batch_cow([0, 1])
    assert len(copies) == 1 and p.num_free == 0
