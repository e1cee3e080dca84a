// Random-operation driver for the host-side bookkeeping (block pool,
// sequences with sharing, fork + copy-on-write, prefix cache, swap, the
// step scheduler) and the fp64 oracle, built with AddressSanitizer and
// UndefinedBehaviorSanitizer by the CPU test that runs it.  It links the
// library's host sources and the oracle's C source directly; no GPU code.
//
// Every step checks the pool's accounting (free + cached + referenced ==
// all blocks; refcounts equal the references the live sequences hold while
// none is swapped out) and every sequence's block count; at the end every
// sequence is released and every block must be back.  Exit status 0 means
// no check failed; the sanitizers abort on the first memory or UB error.
//
//   host_fuzz <seed> <ops>
#include <cstdio>
#include <cstdlib>
#include <map>
#include <random>
#include <set>
#include <vector>

#include "pkv.h"

extern "C" {
int oracle_decode(int B, int Hq, int Hkv, int D, int dtype, const void *q, const void *k,
                  const void *v, const int64_t *seq_start, double scale, double *out,
                  const int32_t *pairs, int npairs, int nthreads);
int oracle_prefill(int S, int Hq, int Hkv, int D, int dtype, const void *q,
                   const int32_t *query_start, const void *k, const void *v,
                   const int64_t *seq_start, double scale, double *out, const int32_t *rows,
                   int nrows, int nthreads);
int oracle_append(const void *k, const void *v, const int32_t *slots, int T, int Hkv, int D,
                  int elem_size, int bs, int64_t num_blocks, void *k_cache, void *v_cache);
int oracle_copy_blocks(const void *src_k, const void *src_v, int64_t src_nb, void *dst_k,
                       void *dst_v, int64_t dst_nb, const int32_t *src_ids,
                       const int32_t *dst_ids, int n, int Hkv, int bs, int D, int elem_size);
}

namespace {

int g_fail = 0;
int g_done[12] = {};        // successful operations per kind (coverage report)
int g_cow = 0;              // copy-on-write copies handed out

#define CHECK(cond)                                                                  \
    do {                                                                             \
        if (!(cond)) {                                                               \
            std::fprintf(stderr, "check failed at line %d: %s\n", __LINE__, #cond);  \
            ++g_fail;                                                                \
        }                                                                            \
    } while (0)

constexpr int32_t kBlocks = 96;
constexpr int32_t kHostBlocks = 48;
constexpr int32_t kBs = 4;

struct World {
    std::mt19937_64 rng;
    pkv_pool *pool = nullptr;
    pkv_pool *host = nullptr;
    pkv_seqs *seqs = nullptr;
    std::map<int64_t, std::vector<int32_t>> prompt;   // token ids of each live sequence
    std::set<int64_t> swapped;
    int64_t next_id = 1;

    int64_t pick()
    {
        if (prompt.empty())
            return -1;
        auto it = prompt.begin();
        std::advance(it, (long)(rng() % prompt.size()));
        return it->first;
    }
    int32_t uni(int32_t lo, int32_t hi) { return lo + (int32_t)(rng() % (uint64_t)(hi - lo + 1)); }
};

void check_accounting(World &w)
{
    int32_t refd = 0;
    std::vector<int32_t> ref(kBlocks, 0);
    for (int32_t id = 0; id < kBlocks; ++id) {
        ref[id] = pkv_pool_refcount(w.pool, id);
        CHECK(ref[id] >= 0);
        refd += ref[id] > 0;
    }
    CHECK(pkv_pool_num_free(w.pool) + refd == kBlocks);
    CHECK(pkv_pool_num_cached(w.pool) <= pkv_pool_num_free(w.pool));
    CHECK(pkv_pool_refcount(w.pool, -1) == -1 && pkv_pool_refcount(w.pool, kBlocks) == -1);
    std::vector<int32_t> held(kBlocks, 0);
    std::vector<int32_t> ids(kBlocks + kHostBlocks);
    for (auto &kv : w.prompt) {
        const int32_t L = pkv_seqs_len(w.seqs, kv.first);
        CHECK(L >= 0);
        const int32_t n = pkv_seqs_block_ids(w.seqs, kv.first, (int32_t)ids.size(), ids.data());
        CHECK(n == (L + kBs - 1) / kBs);
        CHECK(pkv_seqs_is_swapped(w.seqs, kv.first) == (w.swapped.count(kv.first) ? 1 : 0));
        if (w.swapped.count(kv.first))
            continue;
        for (int32_t i = 0; i < n; ++i) {
            CHECK(ids[i] >= 0 && ids[i] < kBlocks);
            if (ids[i] >= 0 && ids[i] < kBlocks)
                ++held[ids[i]];
        }
    }
    if (w.swapped.empty())
        for (int32_t id = 0; id < kBlocks; ++id)
            CHECK(held[id] == ref[id]);
    pkv_seqs_stats st{};
    CHECK(pkv_seqs_stats_get(w.seqs, &st) == PKV_OK);
    CHECK(st.num_seqs == (int32_t)w.prompt.size());
    CHECK(st.blocks_in_use == refd);
}

// One random bookkeeping operation.  Return codes other than OK are legal
// outcomes (exhaustion, sharing rules); the accounting check afterwards is
// what must hold.
void step(World &w)
{
    std::vector<int32_t> slots(64), a(64), b(64);
    int32_t nc = 0;
    const int op = (int)(w.rng() % 12);
    const int64_t s = w.pick();
    switch (op) {
    case 0: {                                   // new sequence from a prompt (prefix cache)
        const int64_t id = w.next_id++;
        std::vector<int32_t> toks(w.uni(1, 24));
        // few distinct token values, so prompts share prefixes often
        for (auto &t : toks)
            t = (int32_t)(w.rng() % 3);
        const int32_t got = pkv_seqs_add_cached(w.seqs, id, toks.data(), (int32_t)toks.size());
        if (got >= 0) {
            CHECK(got % kBs == 0 && got < (int32_t)toks.size());
            w.prompt[id] = toks;
            ++g_done[0];
            const int32_t rest = (int32_t)toks.size() - got;
            if (pkv_seqs_append(w.seqs, id, rest, slots.data()) == PKV_OK && (w.rng() & 1))
                pkv_seqs_cache(w.seqs, id, toks.data(), (int32_t)toks.size());
        }
        break;
    }
    case 1:                                     // plain append of a few tokens
        if (s >= 0 && !w.swapped.count(s)) {
            const int32_t n = w.uni(0, 9);
            if (pkv_seqs_append(w.seqs, s, n, slots.data()) == PKV_OK) {
                ++g_done[1];
                for (int32_t i = 0; i < n; ++i)
                    w.prompt[s].push_back((int32_t)(w.rng() % 3));
            }
        }
        break;
    case 2:                                     // copy-on-write append
        if (s >= 0 && !w.swapped.count(s)) {
            const int32_t n = w.uni(1, 6);
            if (pkv_seqs_append_cow(w.seqs, s, n, slots.data(), a.data(), b.data(), &nc) ==
                PKV_OK) {
                CHECK(nc >= 0 && nc <= 1);
                ++g_done[2];
                g_cow += nc;
                for (int32_t i = 0; i < n; ++i)
                    w.prompt[s].push_back((int32_t)(w.rng() % 3));
            }
        }
        break;
    case 3: {                                   // decode step over several sequences, with CoW
        std::vector<int64_t> ids;
        for (auto &kv : w.prompt)
            if (!w.swapped.count(kv.first) && ids.size() < 32 && (w.rng() & 1))
                ids.push_back(kv.first);
        if (pkv_seqs_append_batch_cow(w.seqs, (int32_t)ids.size(), ids.data(), slots.data(),
                                      a.data(), b.data(), &nc) == PKV_OK) {
            CHECK(nc >= 0 && nc <= (int32_t)ids.size());
            ++g_done[3];
            g_cow += nc;
            for (auto id : ids)
                w.prompt[id].push_back((int32_t)(w.rng() % 3));
        }
        break;
    }
    case 4:                                     // fork (shares the partial last block)
        if (s >= 0 && !w.swapped.count(s)) {
            const int64_t id = w.next_id++;
            if (pkv_seqs_fork(w.seqs, id, s) == PKV_OK) {
                ++g_done[4];
                w.prompt[id] = w.prompt[s];
            }
        }
        break;
    case 5:                                     // share whole leading blocks
        if (s >= 0 && !w.swapped.count(s)) {
            const int64_t id = w.next_id++;
            const int32_t full = (int32_t)w.prompt[s].size() / kBs;
            const int32_t nt = full ? w.uni(0, full) * kBs : 0;
            if (pkv_seqs_add_shared(w.seqs, id, s, nt) == PKV_OK) {
                ++g_done[5];
                w.prompt[id] = std::vector<int32_t>(w.prompt[s].begin(),
                                                    w.prompt[s].begin() + nt);
            }
        }
        break;
    case 6:                                     // register full blocks in the prefix cache
        if (s >= 0 && !w.swapped.count(s) &&
            pkv_seqs_cache(w.seqs, s, w.prompt[s].data(), (int32_t)w.prompt[s].size()) == PKV_OK)
            ++g_done[6];
        break;
    case 7:
    case 8:                                     // release
        if (s >= 0) {
            CHECK(pkv_seqs_release(w.seqs, s) == PKV_OK);
            ++g_done[op];
            w.prompt.erase(s);
            w.swapped.erase(s);
        }
        break;
    case 9:                                     // swap out
        if (s >= 0 && !w.swapped.count(s)) {
            int32_t n = 0;
            std::vector<int32_t> d(kBlocks), h(kBlocks);
            if (pkv_seqs_swap_out(w.seqs, s, w.host, kBlocks, d.data(), h.data(), &n) == PKV_OK) {
                CHECK(n >= 0 && n <= kBlocks);
                ++g_done[9];
                w.swapped.insert(s);
            }
        }
        break;
    case 10:                                    // swap in
        if (!w.swapped.empty()) {
            const int64_t id = *w.swapped.begin();
            int32_t n = 0;
            std::vector<int32_t> d(kBlocks), h(kBlocks);
            if (pkv_seqs_swap_in(w.seqs, id, kBlocks, h.data(), d.data(), &n) == PKV_OK) {
                ++g_done[10];
                w.swapped.erase(id);
            }
        }
        break;
    case 11: {                                  // block tables for the resident sequences
        std::vector<int64_t> ids;
        for (auto &kv : w.prompt)
            if (!w.swapped.count(kv.first))
                ids.push_back(kv.first);
        const int32_t stride = 16;
        std::vector<int32_t> tab(ids.size() * stride + 1), lens(ids.size() + 1);
        const int rc = pkv_seqs_fill(w.seqs, (int32_t)ids.size(), ids.data(), tab.data(), stride,
                                     lens.data());
        CHECK(rc == PKV_OK || rc == PKV_EINVAL);
        g_done[11] += rc == PKV_OK;
        break;
    }
    }
}

void run_bookkeeping(uint64_t seed, int ops)
{
    World w;
    w.rng.seed(seed);
    w.pool = pkv_pool_create(kBlocks, seed | 1);
    w.host = pkv_pool_create(kHostBlocks, 0);
    w.seqs = pkv_seqs_create(w.pool, kBs);
    CHECK(w.pool && w.host && w.seqs);
    for (int i = 0; i < ops; ++i) {
        step(w);
        check_accounting(w);
    }
    // Misuse must be refused, not corrupt anything.
    int32_t bad = kBlocks + 7;
    CHECK(pkv_pool_release(w.pool, 1, &bad) == PKV_ESTATE);
    CHECK(pkv_seqs_release(w.seqs, -12345) != PKV_OK);
    while (!w.prompt.empty()) {
        const int64_t s = w.prompt.begin()->first;
        CHECK(pkv_seqs_release(w.seqs, s) == PKV_OK);
        w.prompt.erase(s);
        w.swapped.erase(s);
    }
    check_accounting(w);
    CHECK(pkv_pool_num_free(w.pool) == kBlocks);
    CHECK(pkv_pool_num_free(w.host) == kHostBlocks);
    for (int32_t id = 0; id < kBlocks; ++id)
        CHECK(pkv_pool_refcount(w.pool, id) == 0);
    pkv_seqs_destroy(w.seqs);
    pkv_pool_destroy(w.host);
    pkv_pool_destroy(w.pool);
}

void run_scheduler(uint64_t seed)
{
    std::mt19937_64 rng(seed);
    const int32_t blocks = 64, budget = 24, chunk = 8, max_running = 6;
    pkv_pool *pool = pkv_pool_create(blocks, seed);
    pkv_seqs *seqs = pkv_seqs_create(pool, kBs);
    pkv_sched *sc = pkv_sched_create(pool, seqs, kBs, budget, chunk, max_running);
    CHECK(pool && seqs && sc);
    std::vector<int64_t> d_ids(max_running), c_ids(max_running), f_ids(max_running),
        fin(max_running), pre(max_running);
    std::vector<int32_t> d_slots(max_running), c_prior(max_running), c_len(max_running),
        c_slots(budget);
    pkv_step_plan plan{};
    plan.decode_ids = d_ids.data();
    plan.decode_slots = d_slots.data();
    plan.chunk_ids = c_ids.data();
    plan.chunk_prior = c_prior.data();
    plan.chunk_len = c_len.data();
    plan.chunk_slots = c_slots.data();
    plan.first_ids = f_ids.data();
    plan.finished_ids = fin.data();
    plan.preempted_ids = pre.data();
    int64_t next = 1;
    int submitted = 0, finished = 0;
    for (int stepno = 0; stepno < 4000; ++stepno) {
        if (submitted < 40 && rng() % 3 == 0) {
            const int32_t p = 1 + (int32_t)(rng() % 40), m = 1 + (int32_t)(rng() % 12);
            CHECK(pkv_sched_submit(sc, next++, p, m) == PKV_OK);
            ++submitted;
        }
        CHECK(pkv_sched_step(sc, &plan) == PKV_OK);
        CHECK(plan.n_decode + plan.n_chunk_tokens <= budget);
        CHECK(plan.n_decode <= max_running && plan.n_chunks <= max_running);
        int32_t tok = 0;
        for (int32_t i = 0; i < plan.n_chunks; ++i) {
            CHECK(c_len[i] >= 1 && c_len[i] <= chunk);
            tok += c_len[i];
        }
        CHECK(tok == plan.n_chunk_tokens);
        finished += plan.n_finished;
        if (submitted == 40 && pkv_sched_num_waiting(sc) == 0 && pkv_sched_num_running(sc) == 0)
            break;
    }
    CHECK(finished == 40);
    CHECK(pkv_sched_step(sc, &plan) == PKV_OK);
    CHECK(pkv_pool_num_free(pool) == blocks);
    pkv_sched_destroy(sc);
    pkv_seqs_destroy(seqs);
    pkv_pool_destroy(pool);
}

// The oracle on small random shapes (bounds of every array it touches are
// what the sanitizers check here; its values are pinned by other tests).
void run_oracle(uint64_t seed)
{
    std::mt19937_64 rng(seed);
    std::normal_distribution<float> nd;
    for (int it = 0; it < 6; ++it) {
        const int Hkv = 1 + (int)(rng() % 2), G = 1 << (rng() % 3), Hq = Hkv * G;
        const int D = 8 * (1 + (int)(rng() % 2)), B = 1 + (int)(rng() % 4), bs = 4;
        std::vector<int64_t> st(B + 1, 0);
        for (int b = 0; b < B; ++b)
            st[b + 1] = st[b] + (int64_t)(rng() % 20);
        const int64_t rows = st[B];
        std::vector<float> q((size_t)B * Hq * D), k((size_t)(rows + 1) * Hkv * D),
            v((size_t)(rows + 1) * Hkv * D);
        for (auto *vec : {&q, &k, &v})
            for (auto &x : *vec)
                x = nd(rng);
        std::vector<double> out((size_t)B * Hq * D);
        CHECK(oracle_decode(B, Hq, Hkv, D, 0, q.data(), k.data(), v.data(), st.data(), 0.3,
                            out.data(), nullptr, 0, 2) == 0);
        // prefill: every sequence's last C_b rows are its chunk
        std::vector<int32_t> qs(B + 1, 0);
        for (int b = 0; b < B; ++b)
            qs[b + 1] = qs[b] + (int32_t)((st[b + 1] - st[b]) / 2);
        std::vector<float> pq((size_t)(qs[B] + 1) * Hq * D);
        for (auto &x : pq)
            x = nd(rng);
        std::vector<double> pout((size_t)(qs[B] + 1) * Hq * D);
        CHECK(oracle_prefill(B, Hq, Hkv, D, 0, pq.data(), qs.data(), k.data(), v.data(),
                             st.data(), 0.3, pout.data(), nullptr, 0, 2) == 0);
        // append + copy into a small cache
        const int nb = 6;
        std::vector<float> kc((size_t)nb * Hkv * bs * D), vc(kc.size());
        const int T = (int)std::min<int64_t>(rows, (int64_t)nb * bs);
        std::vector<int32_t> slots(T + 1);
        for (int t = 0; t < T; ++t)
            slots[t] = (rng() % 5 == 0) ? -1 : t;
        CHECK(oracle_append(k.data(), v.data(), slots.data(), T, Hkv, D, 4, bs, nb, kc.data(),
                            vc.data()) == 0);
        int32_t src[3] = {0, 1, 9}, dst[3] = {5, 4, 2};
        CHECK(oracle_copy_blocks(kc.data(), vc.data(), nb, kc.data(), vc.data(), nb, src, dst, 3,
                                 Hkv, bs, D, 4) == 0);
    }
}

}  // namespace

int main(int argc, char **argv)
{
    const uint64_t seed = argc > 1 ? std::strtoull(argv[1], nullptr, 10) : 1;
    const int ops = argc > 2 ? std::atoi(argv[2]) : 2000;
    run_bookkeeping(seed, ops);
    run_scheduler(seed);
    run_oracle(seed);
    if (g_fail) {
        std::fprintf(stderr, "%d checks failed (seed %llu)\n", g_fail, (unsigned long long)seed);
        return 1;
    }
    std::printf("ok seed %llu ops", (unsigned long long)seed);
    for (int i = 0; i < 12; ++i)
        std::printf(" %d", g_done[i]);
    std::printf(" cow %d\n", g_cow);
    return 0;
}
