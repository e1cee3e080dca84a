"""Host block pool and sequence bookkeeping (CPU only).

Behaviour follows "LLM Inference: KV Cache, Batching & Scheduling",
"PagedAttention and vLLM" (on-demand allocation, a finished request's pages
return to the pool at once) and "The KV cache" warning (running out of KV
memory stalls or preempts: here an all-or-nothing PKV_ENOBLOCKS).
"""
import numpy as np
import pytest

import paged_kv_cache_indirected_amd as pkv


def test_ascending_free_list_without_seed():
    p = pkv.Pool(8, seed=0)
    assert p.alloc(3) == [0, 1, 2]
    assert p.num_free == 5 and p.num_blocks == 8


def test_seeded_order_is_a_deterministic_permutation():
    a = pkv.Pool(100, seed=1234).alloc(100)
    b = pkv.Pool(100, seed=1234).alloc(100)
    c = pkv.Pool(100, seed=99).alloc(100)
    assert a == b and sorted(a) == list(range(100))
    assert a != c and a != list(range(100))


def test_release_returns_blocks_to_back_of_free_list():
    p = pkv.Pool(4)
    ids = p.alloc(2)
    p.release([ids[0]])
    assert p.alloc(2) == [2, 3]
    assert p.alloc(1) == [ids[0]]
    assert p.num_free == 0


def test_exhaustion_is_all_or_nothing():
    p = pkv.Pool(5)
    p.alloc(3)
    with pytest.raises(pkv.PkvError) as e:
        p.alloc(3)
    assert e.value.code == pkv.ENOBLOCKS
    assert p.num_free == 2 and p.alloc(2) == [3, 4]


def test_refcounts_share_and_release():
    p = pkv.Pool(4)
    [a] = p.alloc(1)
    p.share([a, a])
    assert p.refcount(a) == 3
    p.release([a, a])
    assert p.refcount(a) == 1 and p.num_free == 3
    p.release([a])
    assert p.refcount(a) == 0 and p.num_free == 4


def test_bad_share_and_release_leave_pool_unchanged():
    p = pkv.Pool(4)
    [a, b] = p.alloc(2)
    with pytest.raises(pkv.PkvError) as e:
        p.release([a, a])          # more often than held
    assert e.value.code == pkv.ESTATE and p.refcount(a) == 1
    with pytest.raises(pkv.PkvError) as e:
        p.share([a, 3])            # 3 is free
    assert e.value.code == pkv.ESTATE and p.refcount(a) == 1
    with pytest.raises(pkv.PkvError) as e:
        p.release([7])             # unknown id
    assert e.value.code == pkv.ESTATE
    assert p.refcount(99) == -1


def test_seq_append_slots_cross_block_boundaries():
    p = pkv.Pool(16, seed=0)
    s = pkv.Seqs(p, 4)
    s.add(7)
    slots = s.append(7, 6)
    blocks = s.block_ids(7)
    assert len(blocks) == 2
    assert list(slots) == [blocks[0] * 4 + i for i in range(4)] + [blocks[1] * 4 + i for i in range(2)]
    more = s.append_batch([7])
    assert more[0] == blocks[1] * 4 + 2 and s.length(7) == 7


def test_seq_release_returns_every_block_at_once():
    p = pkv.Pool(10, seed=3)
    s = pkv.Seqs(p, 16)
    s.add(1)
    s.append(1, 40)
    assert p.num_free == 7
    s.release(1)
    assert p.num_free == 10 and s.length(1) == -1
    with pytest.raises(pkv.PkvError):
        s.release(1)


def test_batch_append_all_or_nothing():
    p = pkv.Pool(3)
    s = pkv.Seqs(p, 2)
    for i in range(3):
        s.add(i)
        s.append(i, 2)             # each fills one block; pool now empty
    with pytest.raises(pkv.PkvError) as e:
        s.append_batch([0, 1, 2])
    assert e.value.code == pkv.ENOBLOCKS
    assert [s.length(i) for i in range(3)] == [2, 2, 2]


def test_prefix_sharing_and_shared_block_protection():
    p = pkv.Pool(20)
    s = pkv.Seqs(p, 4)
    s.add(0)
    s.append(0, 10)                # 2 full blocks + 2 tokens
    with pytest.raises(pkv.PkvError):
        s.add_shared(1, 0, 6)      # not a whole-block prefix
    s.add_shared(1, 0, 8)
    s.add_shared(2, 0, 8)
    b0 = s.block_ids(0)
    assert s.block_ids(1) == b0[:2] and p.refcount(b0[0]) == 3
    # Sequence 1's next token starts a fresh private block.
    slot = s.append(1, 1)[0]
    assert slot // 4 not in b0
    # A sequence whose partially filled last block is shared may not write it.
    s.add_shared(3, 1, 8)
    s.release(0)
    assert p.refcount(b0[0]) == 3
    s.add(9)
    s.append(9, 3)
    s.add_shared(10, 9, 0)
    st = s.stats()
    assert st["num_seqs"] == 5 and st["tokens"] == 9 + 8 + 8 + 3 + 0


def test_write_into_shared_partial_block_is_rejected():
    p = pkv.Pool(8)
    s = pkv.Seqs(p, 4)
    s.add(0)
    s.append(0, 4)
    s.add_shared(1, 0, 4)
    s.append(1, 2)                 # private block for seq 1
    # Force a shared partial block: share seq 1's blocks via the pool.
    ids = s.block_ids(1)
    p.share([ids[-1]])
    with pytest.raises(pkv.PkvError) as e:
        s.append(1, 1)
    assert e.value.code == pkv.ESTATE
    p.release([ids[-1]])
    s.append(1, 1)
    assert s.length(1) == 7


def test_fill_pads_with_minus_one_and_checks_stride():
    p = pkv.Pool(10)
    s = pkv.Seqs(p, 16)
    s.add(5)
    s.append(5, 33)
    s.add(6)
    tab, lens = s.fill([6, 5], 4)
    assert tab.shape == (2, 4) and list(lens) == [0, 33]
    assert list(tab[0]) == [-1] * 4 and list(tab[1, 3:]) == [-1]
    with pytest.raises(pkv.PkvError):
        s.fill([5], 2)


def test_fragmentation_stats():
    p = pkv.Pool(10)
    s = pkv.Seqs(p, 16)
    s.add(1)
    s.append(1, 17)
    st = s.stats()
    assert st["blocks_in_use"] == 2 and st["slots_unused"] == 15 and st["tokens"] == 17


@pytest.mark.parametrize("cow", [False, True])
def test_batch_append_rejects_a_sequence_listed_twice(cow):
    # A decode step gives each sequence one token; a repeated id is a caller
    # error, refused before anything changes.
    pool = pkv.Pool(64, 3)
    s = pkv.Seqs(pool, 4)
    for i in range(40):
        s.add(i)
        s.append(i, 3)
    free, lens = pool.num_free, [s.length(i) for i in range(40)]
    batch = list(range(40)) + [17]
    with pytest.raises(pkv.PkvError) as e:
        (s.append_batch_cow if cow else s.append_batch)(batch)
    assert e.value.code == pkv.EINVAL and "17" in str(e.value)
    assert pool.num_free == free and [s.length(i) for i in range(40)] == lens
