// Host-side block pool and sequence bookkeeping.
//
// Follows "LLM Inference: KV Cache, Batching & Scheduling", section
// "PagedAttention and vLLM": KV lives in fixed-size blocks, pages are
// allocated on demand and a finished request's pages return to the pool at
// once; and the "LLM Inference Engineering" summary, section 2, with the
// blog post's "The Elegant Fix": sequences with an identical prefix share its
// pages.  Sharing is reference counted; a shared block is read-only.
//
// Single-threaded by contract (one scheduler thread owns a pool).
#include <algorithm>
#include <cstring>
#include <deque>
#include <list>
#include <new>
#include <unordered_map>
#include <vector>

#include "pkv_internal.h"

using pkv::fail;

namespace {
// A block registered in the prefix cache: the token ids it holds and the key
// of the block before it in the sequence (the chain makes a block's key
// depend on the whole prefix, not only on its own tokens).
struct CachedBlock {
    uint64_t key = 0;
    uint64_t parent = 0;
    std::vector<int32_t> tokens;
};
}  // namespace

struct pkv_pool {
    int32_t num_blocks = 0;
    std::vector<int32_t> ref;     // refcount per block, 0 = free or cached-only
    std::deque<int32_t> free_q;   // front is handed out next; released blocks go to the back
    // Prefix cache ("LLM Inference: KV Cache, Batching & Scheduling",
    // "Prefix caching"): full blocks keyed by their token chain.  A cached
    // block whose last reference goes away is kept, unreferenced, in an LRU
    // list and only reused for other data when the free list runs dry.
    std::unordered_map<uint64_t, int32_t> index;     // key -> block
    std::vector<CachedBlock> cached;                 // per block (key 0 = not cached)
    std::list<int32_t> lru;                          // front = least recently released
    std::vector<std::list<int32_t>::iterator> lru_at;
    std::vector<char> in_lru;
};

namespace {

// splitmix64: a small, well-known 64-bit mixing generator (Steele, Lea and
// Flood, 2014) used only to draw the initial free-list order.
uint64_t splitmix64(uint64_t &s)
{
    uint64_t z = (s += 0x9E3779B97F4A7C15ull);
    z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
    z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
    return z ^ (z >> 31);
}

bool valid_id(const pkv_pool *p, int32_t id) { return id >= 0 && id < p->num_blocks; }

}  // namespace

extern "C" pkv_pool *pkv_pool_create(int32_t num_blocks, uint64_t seed)
{
    if (num_blocks <= 0) {
        fail(PKV_EINVAL, "pkv_pool_create: num_blocks must be positive (got %d)", num_blocks);
        return nullptr;
    }
    pkv_pool *p = new (std::nothrow) pkv_pool;
    if (!p)
        return nullptr;
    try {
        p->num_blocks = num_blocks;
        p->ref.assign(num_blocks, 0);
        p->cached.resize(num_blocks);
        p->lru_at.resize(num_blocks);
        p->in_lru.assign(num_blocks, 0);
        std::vector<int32_t> order(num_blocks);
        for (int32_t i = 0; i < num_blocks; ++i)
            order[i] = i;
        if (seed != 0) {
            // Fisher-Yates with an unbiased bounded draw (rejection sampling).
            uint64_t s = seed;
            for (int32_t i = num_blocks - 1; i > 0; --i) {
                uint64_t bound = (uint64_t)i + 1, lim = UINT64_MAX - UINT64_MAX % bound, x;
                do {
                    x = splitmix64(s);
                } while (x >= lim);
                std::swap(order[i], order[(size_t)(x % bound)]);
            }
        }
        p->free_q.assign(order.begin(), order.end());
    } catch (...) {
        delete p;
        return nullptr;
    }
    return p;
}

extern "C" void pkv_pool_destroy(pkv_pool *pool) { delete pool; }

namespace {

void forget(pkv_pool *p, int32_t id)
{
    CachedBlock &c = p->cached[id];
    if (c.key != 0) {
        auto it = p->index.find(c.key);
        if (it != p->index.end() && it->second == id)
            p->index.erase(it);
        c = CachedBlock{};
    }
}

void lru_remove(pkv_pool *p, int32_t id)
{
    if (p->in_lru[id]) {
        p->lru.erase(p->lru_at[id]);
        p->in_lru[id] = 0;
    }
}

}  // namespace

extern "C" int pkv_pool_alloc(pkv_pool *p, int32_t n, int32_t *ids)
{
    if (!p || n < 0 || (n > 0 && !ids))
        return fail(PKV_EINVAL, "pkv_pool_alloc: bad arguments");
    if ((size_t)n > p->free_q.size() + p->lru.size())
        return fail(PKV_ENOBLOCKS, "pkv_pool_alloc: %d blocks requested, %zu free", n,
                    p->free_q.size() + p->lru.size());
    for (int32_t i = 0; i < n; ++i) {
        int32_t id;
        if (!p->free_q.empty()) {
            id = p->free_q.front();
            p->free_q.pop_front();
        } else {   // evict the least recently released cached block
            id = p->lru.front();
            lru_remove(p, id);
            forget(p, id);
        }
        p->ref[id] = 1;
        ids[i] = id;
    }
    return PKV_OK;
}

extern "C" int pkv_pool_share(pkv_pool *p, int32_t n, const int32_t *ids)
{
    if (!p || n < 0 || (n > 0 && !ids))
        return fail(PKV_EINVAL, "pkv_pool_share: bad arguments");
    for (int32_t i = 0; i < n; ++i)
        if (!valid_id(p, ids[i]) || p->ref[ids[i]] == 0)
            return fail(PKV_ESTATE, "pkv_pool_share: block %d is free or unknown", ids[i]);
    for (int32_t i = 0; i < n; ++i)
        ++p->ref[ids[i]];
    return PKV_OK;
}

extern "C" int pkv_pool_release(pkv_pool *p, int32_t n, const int32_t *ids)
{
    if (!p || n < 0 || (n > 0 && !ids))
        return fail(PKV_EINVAL, "pkv_pool_release: bad arguments");
    std::unordered_map<int32_t, int32_t> count;
    for (int32_t i = 0; i < n; ++i) {
        if (!valid_id(p, ids[i]))
            return fail(PKV_ESTATE, "pkv_pool_release: unknown block %d", ids[i]);
        if (++count[ids[i]] > p->ref[ids[i]])
            return fail(PKV_ESTATE, "pkv_pool_release: block %d released more often than held",
                        ids[i]);
    }
    for (int32_t i = 0; i < n; ++i)
        if (--p->ref[ids[i]] == 0) {
            const int32_t id = ids[i];
            if (p->cached[id].key != 0) {
                p->lru_at[id] = p->lru.insert(p->lru.end(), id);
                p->in_lru[id] = 1;
            } else {
                p->free_q.push_back(id);
            }
        }
    return PKV_OK;
}

extern "C" int32_t pkv_pool_num_free(const pkv_pool *p)
{
    return p ? (int32_t)(p->free_q.size() + p->lru.size()) : -1;
}

extern "C" int32_t pkv_pool_num_cached(const pkv_pool *p)
{
    return p ? (int32_t)p->lru.size() : -1;
}

// ---------------------------------------------------------------------------
// Prefix cache.

namespace {

constexpr uint64_t kChainSeed = 0x243F6A8885A308D3ull;   // key "before" the first block

// Key of a block from its parent's key and its token ids: 64-bit FNV-1a over
// the parent key's and the tokens' bytes, forced non-zero (0 marks "not
// cached").  Collisions are caught on lookup by comparing the stored tokens
// and parent key.
uint64_t block_key(uint64_t parent, const int32_t *toks, int32_t bs)
{
    uint64_t h = 0xCBF29CE484222325ull;
    auto mix = [&](uint64_t v, int nbytes) {
        for (int i = 0; i < nbytes; ++i) {
            h ^= (v >> (8 * i)) & 0xFF;
            h *= 0x100000001B3ull;
        }
    };
    mix(parent, 8);
    for (int32_t i = 0; i < bs; ++i)
        mix((uint32_t)toks[i], 4);
    return h ? h : 1;
}

bool holds(const pkv_pool *p, int32_t id, uint64_t parent, const int32_t *toks, int32_t bs)
{
    const CachedBlock &c = p->cached[id];
    return c.parent == parent && (int32_t)c.tokens.size() == bs &&
           std::equal(c.tokens.begin(), c.tokens.end(), toks);
}

// Longest run of cached blocks holding tokens[0 .. k*bs), k <= cap; each
// found block gains a reference (and leaves the LRU list).  Returns k.
int32_t prefix_match(pkv_pool *p, int32_t block_size, const int32_t *tokens, int32_t n,
                     int32_t *ids, int32_t cap)
{
    int32_t k = 0;
    uint64_t parent = kChainSeed;
    for (; k < cap && (int64_t)(k + 1) * block_size <= n; ++k) {
        const int32_t *t = tokens + (int64_t)k * block_size;
        const uint64_t key = block_key(parent, t, block_size);
        auto it = p->index.find(key);
        if (it == p->index.end() || !holds(p, it->second, parent, t, block_size))
            break;
        ids[k] = it->second;
        parent = key;
    }
    for (int32_t i = 0; i < k; ++i) {
        lru_remove(p, ids[i]);
        ++p->ref[ids[i]];
    }
    return k;
}

// Register blocks ids[0 .. n/bs) (allocated) as holding tokens[0 .. n/bs*bs).
void prefix_insert(pkv_pool *p, int32_t block_size, const int32_t *tokens, int32_t n,
                   const int32_t *ids)
{
    const int32_t nb = n / block_size;
    uint64_t parent = kChainSeed;
    for (int32_t i = 0; i < nb; ++i) {
        const int32_t *t = tokens + (int64_t)i * block_size;
        const uint64_t key = block_key(parent, t, block_size);
        auto it = p->index.find(key);
        if (it == p->index.end()) {
            // A block can hold one cached identity; re-registering it under
            // another chain replaces the old entry.
            forget(p, ids[i]);
            p->index.emplace(key, ids[i]);
            CachedBlock &c = p->cached[ids[i]];
            c.key = key;
            c.parent = parent;
            c.tokens.assign(t, t + block_size);
        }
        parent = key;
    }
}

}  // namespace

extern "C" int32_t pkv_pool_num_blocks(const pkv_pool *p) { return p ? p->num_blocks : -1; }

extern "C" int32_t pkv_pool_refcount(const pkv_pool *p, int32_t id)
{
    return (p && valid_id(p, id)) ? p->ref[id] : -1;
}

// ---------------------------------------------------------------------------
// Sequences.

namespace {
struct Seq {
    int32_t len = 0;
    std::vector<int32_t> blocks;
    // Swapped out: on_host[i] says blocks[i] is a slot of the host pool
    // `host` (blocks the sequence held alone); shared blocks stay resident.
    std::vector<char> on_host;
    pkv_pool *host = nullptr;
    bool swapped() const { return host != nullptr; }
};
}  // namespace

struct pkv_seqs {
    pkv_pool *pool = nullptr;
    int32_t bs = 0;
    std::unordered_map<int64_t, Seq> seqs;
};

extern "C" pkv_seqs *pkv_seqs_create(pkv_pool *pool, int32_t block_size)
{
    if (!pool || block_size <= 0) {
        fail(PKV_EINVAL, "pkv_seqs_create: bad arguments");
        return nullptr;
    }
    pkv_seqs *s = new (std::nothrow) pkv_seqs;
    if (!s)
        return nullptr;
    s->pool = pool;
    s->bs = block_size;
    return s;
}

extern "C" void pkv_seqs_destroy(pkv_seqs *s) { delete s; }

extern "C" int pkv_seqs_add(pkv_seqs *s, int64_t id)
{
    if (!s)
        return fail(PKV_EINVAL, "pkv_seqs_add: null handle");
    if (s->seqs.count(id))
        return fail(PKV_ESTATE, "pkv_seqs_add: sequence %lld exists", (long long)id);
    s->seqs.emplace(id, Seq{});
    return PKV_OK;
}

extern "C" int pkv_seqs_add_shared(pkv_seqs *s, int64_t id, int64_t src, int32_t num_tokens)
{
    if (!s)
        return fail(PKV_EINVAL, "pkv_seqs_add_shared: null handle");
    auto it = s->seqs.find(src);
    if (it == s->seqs.end())
        return fail(PKV_ESTATE, "pkv_seqs_add_shared: unknown source %lld", (long long)src);
    if (it->second.swapped())
        return fail(PKV_ESTATE, "pkv_seqs_add_shared: source %lld is swapped out", (long long)src);
    if (s->seqs.count(id))
        return fail(PKV_ESTATE, "pkv_seqs_add_shared: sequence %lld exists", (long long)id);
    if (num_tokens < 0 || num_tokens % s->bs != 0 || num_tokens > it->second.len)
        return fail(PKV_EINVAL,
                    "pkv_seqs_add_shared: %d tokens is not a whole-block prefix of a %d-token "
                    "sequence",
                    num_tokens, it->second.len);
    Seq n;
    n.len = num_tokens;
    n.blocks.assign(it->second.blocks.begin(), it->second.blocks.begin() + num_tokens / s->bs);
    int rc = pkv_pool_share(s->pool, (int32_t)n.blocks.size(), n.blocks.data());
    if (rc != PKV_OK)
        return rc;
    s->seqs.emplace(id, std::move(n));
    return PKV_OK;
}

extern "C" int pkv_seqs_fork(pkv_seqs *s, int64_t id, int64_t src)
{
    if (!s)
        return fail(PKV_EINVAL, "pkv_seqs_fork: null handle");
    auto it = s->seqs.find(src);
    if (it == s->seqs.end())
        return fail(PKV_ESTATE, "pkv_seqs_fork: unknown source %lld", (long long)src);
    if (it->second.swapped())
        return fail(PKV_ESTATE, "pkv_seqs_fork: source %lld is swapped out", (long long)src);
    if (s->seqs.count(id))
        return fail(PKV_ESTATE, "pkv_seqs_fork: sequence %lld exists", (long long)id);
    Seq n = it->second;
    int rc = pkv_pool_share(s->pool, (int32_t)n.blocks.size(), n.blocks.data());
    if (rc != PKV_OK)
        return rc;
    s->seqs.emplace(id, std::move(n));
    return PKV_OK;
}

extern "C" int32_t pkv_seqs_add_cached(pkv_seqs *s, int64_t id, const int32_t *tokens, int32_t n)
{
    if (!s || n < 0 || (n > 0 && !tokens))
        return fail(PKV_EINVAL, "pkv_seqs_add_cached: bad arguments");
    if (s->seqs.count(id))
        return fail(PKV_ESTATE, "pkv_seqs_add_cached: sequence %lld exists", (long long)id);
    // At least one token is left to compute, so the prompt's last position
    // always gets a fresh query.
    const int32_t cap = n > 0 ? (n - 1) / s->bs : 0;
    Seq q;
    q.blocks.resize(cap);
    const int32_t k = prefix_match(s->pool, s->bs, tokens, n, q.blocks.data(), cap);
    q.blocks.resize(k);
    q.len = k * s->bs;
    s->seqs.emplace(id, std::move(q));
    return k * s->bs;
}

extern "C" int pkv_seqs_cache(pkv_seqs *s, int64_t id, const int32_t *tokens, int32_t n)
{
    if (!s || n < 0 || (n > 0 && !tokens))
        return fail(PKV_EINVAL, "pkv_seqs_cache: bad arguments");
    auto it = s->seqs.find(id);
    if (it == s->seqs.end())
        return fail(PKV_ESTATE, "pkv_seqs_cache: unknown sequence %lld", (long long)id);
    if (it->second.swapped())
        return fail(PKV_ESTATE, "pkv_seqs_cache: sequence %lld is swapped out", (long long)id);
    if (n > it->second.len)
        return fail(PKV_EINVAL, "pkv_seqs_cache: %d tokens given for a %d-token sequence", n,
                    it->second.len);
    prefix_insert(s->pool, s->bs, tokens, n, it->second.blocks.data());
    return PKV_OK;
}

namespace {

// Blocks a sequence of `len` tokens must gain to hold `len + n`.
int32_t blocks_needed(const Seq &q, int32_t bs, int32_t n)
{
    int64_t need = ((int64_t)q.len + n + bs - 1) / bs;
    return (int32_t)std::max<int64_t>(0, need - (int64_t)q.blocks.size());
}

// The first id listed more than once in ids[0..n), or -1 (a sorted copy:
// O(n log n) for the batch of a decode step).
int64_t first_duplicate(int32_t n, const int64_t *ids, bool *found)
{
    std::vector<int64_t> v(ids, ids + n);
    std::sort(v.begin(), v.end());
    for (int32_t i = 1; i < n; ++i)
        if (v[i] == v[i - 1]) {
            *found = true;
            return v[i];
        }
    *found = false;
    return -1;
}

// Appending into the partially filled last block is only allowed when that
// block is private.
bool writes_shared_block(const pkv_seqs *s, const Seq &q, int32_t n)
{
    if (n <= 0 || q.len % s->bs == 0 || q.blocks.empty())
        return false;
    return pkv_pool_refcount(s->pool, q.blocks.back()) > 1;
}

void take_slots(const pkv_seqs *s, Seq &q, int32_t n, int32_t *slots)
{
    for (int32_t i = 0; i < n; ++i) {
        int32_t pos = q.len + i;
        slots[i] = q.blocks[pos / s->bs] * s->bs + pos % s->bs;
    }
    q.len += n;
}

}  // namespace

extern "C" int pkv_seqs_append(pkv_seqs *s, int64_t id, int32_t n, int32_t *slots)
{
    if (!s || n < 0 || (n > 0 && !slots))
        return fail(PKV_EINVAL, "pkv_seqs_append: bad arguments");
    auto it = s->seqs.find(id);
    if (it == s->seqs.end())
        return fail(PKV_ESTATE, "pkv_seqs_append: unknown sequence %lld", (long long)id);
    Seq &q = it->second;
    if (q.swapped())
        return fail(PKV_ESTATE, "pkv_seqs_append: sequence %lld is swapped out", (long long)id);
    if ((int64_t)q.len + n > INT32_MAX / 2)
        return fail(PKV_EINVAL, "pkv_seqs_append: sequence too long");
    if (writes_shared_block(s, q, n))
        return fail(PKV_ESTATE, "pkv_seqs_append: sequence %lld would write into a shared block",
                    (long long)id);
    int32_t nb = blocks_needed(q, s->bs, n);
    std::vector<int32_t> fresh(nb);
    int rc = pkv_pool_alloc(s->pool, nb, fresh.data());
    if (rc != PKV_OK)
        return rc;
    q.blocks.insert(q.blocks.end(), fresh.begin(), fresh.end());
    take_slots(s, q, n, slots);
    return PKV_OK;
}

extern "C" int pkv_seqs_append_batch(pkv_seqs *s, int32_t n, const int64_t *ids, int32_t *slots)
{
    if (!s || n < 0 || (n > 0 && (!ids || !slots)))
        return fail(PKV_EINVAL, "pkv_seqs_append_batch: bad arguments");
    bool dup = false;
    const int64_t d = first_duplicate(n, ids, &dup);
    if (dup)
        return fail(PKV_EINVAL, "pkv_seqs_append_batch: sequence %lld listed twice", (long long)d);
    std::vector<Seq *> qs(n);
    int32_t total = 0;
    for (int32_t i = 0; i < n; ++i) {
        auto it = s->seqs.find(ids[i]);
        if (it == s->seqs.end())
            return fail(PKV_ESTATE, "pkv_seqs_append_batch: unknown sequence %lld",
                        (long long)ids[i]);
        qs[i] = &it->second;
        if (qs[i]->swapped())
            return fail(PKV_ESTATE, "pkv_seqs_append_batch: sequence %lld is swapped out",
                        (long long)ids[i]);
        if (writes_shared_block(s, *qs[i], 1))
            return fail(PKV_ESTATE,
                        "pkv_seqs_append_batch: sequence %lld would write into a shared block",
                        (long long)ids[i]);
        total += blocks_needed(*qs[i], s->bs, 1);
    }
    std::vector<int32_t> fresh(total);
    int rc = pkv_pool_alloc(s->pool, total, fresh.data());
    if (rc != PKV_OK)
        return rc;
    int32_t k = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (blocks_needed(*qs[i], s->bs, 1))
            qs[i]->blocks.push_back(fresh[k++]);
        take_slots(s, *qs[i], 1, slots + i);
    }
    return PKV_OK;
}

namespace {

// Give sequence q a private copy of its shared, partially filled last block:
// `fresh` replaces it in q's list and q's reference to the old block drops
// (the old block stays allocated: other sequences still hold it).
void cow_last(pkv_seqs *s, Seq &q, int32_t fresh, int32_t *src, int32_t *dst)
{
    const int32_t old = q.blocks.back();
    q.blocks.back() = fresh;
    pkv_pool_release(s->pool, 1, &old);
    *src = old;
    *dst = fresh;
}

}  // namespace

extern "C" int pkv_seqs_append_cow(pkv_seqs *s, int64_t id, int32_t n, int32_t *slots,
                                   int32_t *copy_src, int32_t *copy_dst, int32_t *num_copies)
{
    if (!s || n < 0 || (n > 0 && !slots) || !copy_src || !copy_dst || !num_copies)
        return fail(PKV_EINVAL, "pkv_seqs_append_cow: bad arguments");
    auto it = s->seqs.find(id);
    if (it == s->seqs.end())
        return fail(PKV_ESTATE, "pkv_seqs_append_cow: unknown sequence %lld", (long long)id);
    Seq &q = it->second;
    if (q.swapped())
        return fail(PKV_ESTATE, "pkv_seqs_append_cow: sequence %lld is swapped out", (long long)id);
    if ((int64_t)q.len + n > INT32_MAX / 2)
        return fail(PKV_EINVAL, "pkv_seqs_append_cow: sequence too long");
    const bool cow = writes_shared_block(s, q, n);
    const int32_t nb = blocks_needed(q, s->bs, n);
    std::vector<int32_t> fresh(nb + (cow ? 1 : 0));
    int rc = pkv_pool_alloc(s->pool, (int32_t)fresh.size(), fresh.data());
    if (rc != PKV_OK)
        return rc;
    *num_copies = 0;
    if (cow) {
        cow_last(s, q, fresh.back(), copy_src, copy_dst);
        *num_copies = 1;
    }
    q.blocks.insert(q.blocks.end(), fresh.begin(), fresh.begin() + nb);
    take_slots(s, q, n, slots);
    return PKV_OK;
}

extern "C" int pkv_seqs_append_batch_cow(pkv_seqs *s, int32_t n, const int64_t *ids, int32_t *slots,
                                         int32_t *copy_src, int32_t *copy_dst,
                                         int32_t *num_copies)
{
    if (!s || n < 0 || (n > 0 && (!ids || !slots || !copy_src || !copy_dst)) || !num_copies)
        return fail(PKV_EINVAL, "pkv_seqs_append_batch_cow: bad arguments");
    bool dup = false;
    const int64_t d = first_duplicate(n, ids, &dup);
    if (dup)
        return fail(PKV_EINVAL, "pkv_seqs_append_batch_cow: sequence %lld listed twice",
                    (long long)d);
    std::vector<Seq *> qs(n);
    std::unordered_map<int32_t, int32_t> sharers;   // shared partial last block -> batch sharers
    int32_t total = 0;
    for (int32_t i = 0; i < n; ++i) {
        auto it = s->seqs.find(ids[i]);
        if (it == s->seqs.end())
            return fail(PKV_ESTATE, "pkv_seqs_append_batch_cow: unknown sequence %lld",
                        (long long)ids[i]);
        qs[i] = &it->second;
        if (qs[i]->swapped())
            return fail(PKV_ESTATE, "pkv_seqs_append_batch_cow: sequence %lld is swapped out",
                        (long long)ids[i]);
        if (writes_shared_block(s, *qs[i], 1))
            ++sharers[qs[i]->blocks.back()];
        total += blocks_needed(*qs[i], s->bs, 1);
    }
    // Copies are decided in batch order.  When every holder of a shared block
    // is in the batch, the last of them to reach it keeps the original.
    for (const auto &kv : sharers)
        total += kv.second - (pkv_pool_refcount(s->pool, kv.first) == kv.second ? 1 : 0);
    std::vector<int32_t> fresh(total);
    int rc = pkv_pool_alloc(s->pool, total, fresh.data());
    if (rc != PKV_OK)
        return rc;
    int32_t k = 0, c = 0;
    for (int32_t i = 0; i < n; ++i) {
        if (writes_shared_block(s, *qs[i], 1)) {
            cow_last(s, *qs[i], fresh[k++], copy_src + c, copy_dst + c);
            ++c;
        }
        if (blocks_needed(*qs[i], s->bs, 1))
            qs[i]->blocks.push_back(fresh[k++]);
        take_slots(s, *qs[i], 1, slots + i);
    }
    *num_copies = c;
    return PKV_OK;
}

extern "C" int pkv_seqs_release(pkv_seqs *s, int64_t id)
{
    if (!s)
        return fail(PKV_EINVAL, "pkv_seqs_release: null handle");
    auto it = s->seqs.find(id);
    if (it == s->seqs.end())
        return fail(PKV_ESTATE, "pkv_seqs_release: unknown sequence %lld", (long long)id);
    Seq &q = it->second;
    if (q.swapped()) {
        std::vector<int32_t> dev, host;
        for (size_t i = 0; i < q.blocks.size(); ++i)
            (q.on_host[i] ? host : dev).push_back(q.blocks[i]);
        int rc = pkv_pool_release(s->pool, (int32_t)dev.size(), dev.data());
        if (rc != PKV_OK)
            return rc;
        rc = pkv_pool_release(q.host, (int32_t)host.size(), host.data());
        if (rc != PKV_OK)
            return rc;
    } else {
        int rc = pkv_pool_release(s->pool, (int32_t)q.blocks.size(), q.blocks.data());
        if (rc != PKV_OK)
            return rc;
    }
    s->seqs.erase(it);
    return PKV_OK;
}

// ---------------------------------------------------------------------------
// Swap (preemption under KV pressure: "LLM Inference: KV Cache, Batching &
// Scheduling", section "The KV cache", which warns that running out of KV
// memory stalls new requests or forces preemption of running ones).

extern "C" int pkv_seqs_swap_out(pkv_seqs *s, int64_t id, pkv_pool *host, int32_t cap,
                                 int32_t *dev_ids, int32_t *host_ids, int32_t *n)
{
    if (!s || !host || host == s->pool || cap < 0 || !n || (cap > 0 && (!dev_ids || !host_ids)))
        return fail(PKV_EINVAL, "pkv_seqs_swap_out: bad arguments");
    auto it = s->seqs.find(id);
    if (it == s->seqs.end())
        return fail(PKV_ESTATE, "pkv_seqs_swap_out: unknown sequence %lld", (long long)id);
    Seq &q = it->second;
    if (q.swapped())
        return fail(PKV_ESTATE, "pkv_seqs_swap_out: sequence %lld is already swapped out",
                    (long long)id);
    // Blocks the sequence holds alone move; shared ones stay resident.
    std::vector<size_t> mine;
    for (size_t i = 0; i < q.blocks.size(); ++i)
        if (pkv_pool_refcount(s->pool, q.blocks[i]) == 1)
            mine.push_back(i);
    if ((int64_t)mine.size() > cap)
        return fail(PKV_EINVAL, "pkv_seqs_swap_out: %zu blocks move, room for %d", mine.size(),
                    cap);
    std::vector<int32_t> slots(mine.size());
    int rc = pkv_pool_alloc(host, (int32_t)slots.size(), slots.data());
    if (rc != PKV_OK)
        return rc;
    std::vector<int32_t> freed(mine.size());
    q.on_host.assign(q.blocks.size(), 0);
    for (size_t k = 0; k < mine.size(); ++k) {
        const size_t i = mine[k];
        dev_ids[k] = freed[k] = q.blocks[i];
        host_ids[k] = slots[k];
        q.blocks[i] = slots[k];
        q.on_host[i] = 1;
    }
    q.host = host;
    pkv_pool_release(s->pool, (int32_t)freed.size(), freed.data());
    *n = (int32_t)mine.size();
    return PKV_OK;
}

extern "C" int pkv_seqs_swap_in(pkv_seqs *s, int64_t id, int32_t cap, int32_t *host_ids,
                                int32_t *dev_ids, int32_t *n)
{
    if (!s || cap < 0 || !n || (cap > 0 && (!dev_ids || !host_ids)))
        return fail(PKV_EINVAL, "pkv_seqs_swap_in: bad arguments");
    auto it = s->seqs.find(id);
    if (it == s->seqs.end())
        return fail(PKV_ESTATE, "pkv_seqs_swap_in: unknown sequence %lld", (long long)id);
    Seq &q = it->second;
    if (!q.swapped())
        return fail(PKV_ESTATE, "pkv_seqs_swap_in: sequence %lld is resident", (long long)id);
    std::vector<size_t> away;
    for (size_t i = 0; i < q.blocks.size(); ++i)
        if (q.on_host[i])
            away.push_back(i);
    if ((int64_t)away.size() > cap)
        return fail(PKV_EINVAL, "pkv_seqs_swap_in: %zu blocks move, room for %d", away.size(),
                    cap);
    std::vector<int32_t> fresh(away.size());
    int rc = pkv_pool_alloc(s->pool, (int32_t)fresh.size(), fresh.data());
    if (rc != PKV_OK)
        return rc;
    std::vector<int32_t> slots(away.size());
    for (size_t k = 0; k < away.size(); ++k) {
        const size_t i = away[k];
        host_ids[k] = slots[k] = q.blocks[i];
        dev_ids[k] = fresh[k];
        q.blocks[i] = fresh[k];
    }
    pkv_pool_release(q.host, (int32_t)slots.size(), slots.data());
    q.host = nullptr;
    q.on_host.clear();
    *n = (int32_t)away.size();
    return PKV_OK;
}

extern "C" int pkv_seqs_is_swapped(const pkv_seqs *s, int64_t id)
{
    if (!s)
        return -1;
    auto it = s->seqs.find(id);
    return it == s->seqs.end() ? -1 : (it->second.swapped() ? 1 : 0);
}

extern "C" int32_t pkv_seqs_len(const pkv_seqs *s, int64_t id)
{
    if (!s)
        return -1;
    auto it = s->seqs.find(id);
    return it == s->seqs.end() ? -1 : it->second.len;
}

extern "C" int32_t pkv_seqs_block_ids(const pkv_seqs *s, int64_t id, int32_t cap, int32_t *ids)
{
    if (!s || cap < 0 || (cap > 0 && !ids))
        return fail(PKV_EINVAL, "pkv_seqs_block_ids: bad arguments");
    auto it = s->seqs.find(id);
    if (it == s->seqs.end())
        return fail(PKV_ESTATE, "pkv_seqs_block_ids: unknown sequence %lld", (long long)id);
    const auto &b = it->second.blocks;
    int32_t n = std::min<int32_t>(cap, (int32_t)b.size());
    if (n > 0)
        std::memcpy(ids, b.data(), sizeof(int32_t) * n);
    return (int32_t)b.size();
}

extern "C" int pkv_seqs_fill(const pkv_seqs *s, int32_t n, const int64_t *ids, int32_t *tables,
                             int32_t stride, int32_t *lens)
{
    if (!s || n < 0 || stride <= 0 || (n > 0 && (!ids || !tables || !lens)))
        return fail(PKV_EINVAL, "pkv_seqs_fill: bad arguments");
    for (int32_t i = 0; i < n; ++i) {
        auto it = s->seqs.find(ids[i]);
        if (it == s->seqs.end())
            return fail(PKV_ESTATE, "pkv_seqs_fill: unknown sequence %lld", (long long)ids[i]);
        if (it->second.swapped())
            return fail(PKV_ESTATE, "pkv_seqs_fill: sequence %lld is swapped out",
                        (long long)ids[i]);
        if ((int64_t)it->second.blocks.size() > stride)
            return fail(PKV_EINVAL, "pkv_seqs_fill: sequence %lld has %zu blocks > stride %d",
                        (long long)ids[i], it->second.blocks.size(), stride);
    }
    for (int32_t i = 0; i < n; ++i) {
        const Seq &q = s->seqs.find(ids[i])->second;
        int32_t *row = tables + (int64_t)i * stride;
        std::fill(row, row + stride, -1);
        std::copy(q.blocks.begin(), q.blocks.end(), row);
        lens[i] = q.len;
    }
    return PKV_OK;
}

extern "C" int pkv_seqs_stats_get(const pkv_seqs *s, pkv_seqs_stats *out)
{
    if (!s || !out)
        return fail(PKV_EINVAL, "pkv_seqs_stats_get: bad arguments");
    pkv_seqs_stats st{};
    st.num_seqs = (int32_t)s->seqs.size();
    for (const auto &kv : s->seqs) {
        st.blocks_referenced += (int64_t)kv.second.blocks.size();
        st.tokens += kv.second.len;
        st.slots_unused += (int64_t)kv.second.blocks.size() * s->bs - kv.second.len;
    }
    st.blocks_in_use = pkv_pool_num_blocks(s->pool) - pkv_pool_num_free(s->pool);
    *out = st;
    return PKV_OK;
}
