// Token-budget step scheduler over a block pool and its sequences.
//
// Follows "LLM Inference: KV Cache, Batching & Scheduling", sections
// "Continuous batching (Orca)" (sequences join and leave the batch at every
// step) and "Chunked prefill" (a long prompt is split into fixed-size chunks,
// e.g. 512 tokens, that share steps with decode tokens: smoother per-step
// latency at the cost of a slightly later first token), and the warning in
// "The KV cache" (when KV memory runs out, new requests stall or running ones
// are preempted).
//
// Policy of one step, under a budget of B tokens:
//   1. sequences that finished in the previous step are released (not
//      earlier: that step's kernels still read their blocks);
//   2. every running sequence whose prompt is complete gets one decode
//      token, in admission order;
//   3. the rest of the budget goes to prefill chunks of at most C tokens:
//      first to running sequences whose prompt is incomplete, then to new
//      requests admitted first-come first-served (preempted ones first);
//   4. blocks are counted before anything is allocated.  If the pool is
//      short, the newest chunk of a not-yet-admitted request is dropped
//      (it stalls in the queue); if running sequences alone do not fit, the
//      most recently admitted one is preempted by recompute: its blocks are
//      released and it returns to the front of the queue with its progress
//      reset.  The plan is then allocated in one pass that cannot fail.
// Single-threaded, like the pool.
#include <algorithm>
#include <deque>
#include <new>
#include <vector>

#include "pkv_internal.h"

using pkv::fail;

namespace {

struct Req {
    int64_t id = 0;
    int32_t prompt = 0;       // prompt tokens
    int32_t max_new = 1;      // tokens to generate (the first comes with the prompt's end)
    int32_t prefilled = 0;    // prompt tokens whose KV is in the cache
    int32_t generated = 0;    // tokens generated so far
};

}  // namespace

struct pkv_sched {
    pkv_pool *pool = nullptr;
    pkv_seqs *seqs = nullptr;
    int32_t bs = 0, budget = 0, chunk = 0, max_running = 0;
    std::deque<Req> waiting;          // front is admitted next
    std::vector<Req> running;         // admission order
    std::vector<int64_t> to_release;  // finished in the previous step
};

extern "C" pkv_sched *pkv_sched_create(pkv_pool *pool, pkv_seqs *seqs, int32_t block_size,
                                       int32_t token_budget, int32_t chunk_tokens,
                                       int32_t max_running)
{
    if (!pool || !seqs || block_size <= 0 || token_budget <= 0 || chunk_tokens <= 0 ||
        max_running <= 0) {
        fail(PKV_EINVAL, "pkv_sched_create: bad arguments");
        return nullptr;
    }
    pkv_sched *s = new (std::nothrow) pkv_sched;
    if (!s)
        return nullptr;
    s->pool = pool;
    s->seqs = seqs;
    s->bs = block_size;
    s->budget = token_budget;
    s->chunk = chunk_tokens;
    s->max_running = max_running;
    return s;
}

extern "C" void pkv_sched_destroy(pkv_sched *s) { delete s; }

extern "C" int pkv_sched_submit(pkv_sched *s, int64_t req_id, int32_t prompt_len,
                                int32_t max_new_tokens)
{
    if (!s || prompt_len <= 0 || max_new_tokens <= 0)
        return fail(PKV_EINVAL, "pkv_sched_submit: bad arguments");
    if (pkv_seqs_len(s->seqs, req_id) >= 0)
        return fail(PKV_ESTATE, "pkv_sched_submit: id %lld is in use", (long long)req_id);
    for (const Req &r : s->waiting)
        if (r.id == req_id)
            return fail(PKV_ESTATE, "pkv_sched_submit: id %lld is queued", (long long)req_id);
    Req r;
    r.id = req_id;
    r.prompt = prompt_len;
    r.max_new = max_new_tokens;
    s->waiting.push_back(r);
    return PKV_OK;
}

extern "C" int32_t pkv_sched_num_waiting(const pkv_sched *s)
{
    return s ? (int32_t)s->waiting.size() : -1;
}

extern "C" int32_t pkv_sched_num_running(const pkv_sched *s)
{
    return s ? (int32_t)s->running.size() : -1;
}

namespace {

// One entry of the step being planned: sequence index in `running` (or -1
// for a request still in the queue, taken from waiting[q]) and its tokens.
struct Item {
    int run = -1;
    int q = -1;
    int32_t n = 0;            // tokens this step
    bool decode = false;
};

int32_t blocks_for(const pkv_sched *s, int64_t id, int32_t n)
{
    const int32_t len = std::max(0, pkv_seqs_len(s->seqs, id));
    const int32_t have = std::max(0, pkv_seqs_block_ids(s->seqs, id, 0, nullptr));
    const int64_t need = ((int64_t)len + n + s->bs - 1) / s->bs;
    return (int32_t)std::max<int64_t>(0, need - have);
}

}  // namespace

extern "C" int pkv_sched_step(pkv_sched *s, pkv_step_plan *p)
{
    if (!s || !p)
        return fail(PKV_EINVAL, "pkv_sched_step: bad arguments");
    p->n_decode = p->n_chunks = p->n_chunk_tokens = 0;
    p->n_first = p->n_finished = p->n_preempted = 0;

    // 1. Release what finished in the previous step.
    for (int64_t id : s->to_release)
        pkv_seqs_release(s->seqs, id);
    s->to_release.clear();

    std::vector<int64_t> preempted;
    std::vector<Item> plan;
    for (;;) {
        plan.clear();
        int32_t left = s->budget;
        // 2. Decode tokens.
        for (int i = 0; i < (int)s->running.size() && left > 0; ++i) {
            const Req &r = s->running[i];
            if (r.prefilled == r.prompt) {
                plan.push_back({i, -1, 1, true});
                --left;
            }
        }
        // 3. Prefill chunks: running first, then admissions.
        for (int i = 0; i < (int)s->running.size() && left > 0; ++i) {
            const Req &r = s->running[i];
            if (r.prefilled < r.prompt) {
                const int32_t n = std::min({s->chunk, r.prompt - r.prefilled, left});
                plan.push_back({i, -1, n, false});
                left -= n;
            }
        }
        int admitted = 0;
        for (int qi = 0; qi < (int)s->waiting.size() && left > 0 &&
                         (int)s->running.size() + admitted < s->max_running;
             ++qi, ++admitted) {
            const Req &r = s->waiting[qi];
            const int32_t n = std::min({s->chunk, r.prompt, left});
            plan.push_back({-1, qi, n, false});
            left -= n;
        }
        // 4. Blocks: drop new admissions from the back, then preempt.
        int64_t need = 0;
        for (const Item &it : plan)
            need += it.run >= 0 ? blocks_for(s, s->running[it.run].id, it.n)
                                : (it.n + s->bs - 1) / s->bs;
        const int64_t free_blocks = pkv_pool_num_free(s->pool);
        while (need > free_blocks && !plan.empty() && plan.back().run < 0) {
            need -= (plan.back().n + s->bs - 1) / s->bs;
            plan.pop_back();
        }
        if (need <= free_blocks)
            break;
        // Running sequences alone do not fit: preempt the newest by
        // recompute and plan again.
        Req victim = s->running.back();
        s->running.pop_back();
        pkv_seqs_release(s->seqs, victim.id);
        preempted.push_back(victim.id);
        victim.prefilled = 0;
        victim.generated = 0;
        s->waiting.push_front(victim);
        // Terminates: each pass either fits or removes a running sequence,
        // and a plan of admissions only always fits once they are dropped.
    }

    // Admit the planned new requests (they are the first ones of the queue).
    int n_new = 0;
    for (const Item &it : plan)
        if (it.run < 0)
            ++n_new;
    const int base = (int)s->running.size();
    for (int k = 0; k < n_new; ++k) {
        Req r = s->waiting.front();
        s->waiting.pop_front();
        int rc = pkv_seqs_add(s->seqs, r.id);
        if (rc != PKV_OK)
            return rc;
        s->running.push_back(r);
    }
    int next_new = base;
    for (Item &it : plan)
        if (it.run < 0)
            it.run = next_new++;

    // Allocate in plan order: decode tokens first, then chunks.
    for (const Item &it : plan) {
        Req &r = s->running[it.run];
        if (it.decode) {
            const int i = p->n_decode++;
            p->decode_ids[i] = r.id;
            int rc = pkv_seqs_append(s->seqs, r.id, 1, p->decode_slots + i);
            if (rc != PKV_OK)
                return rc;
            if (++r.generated >= r.max_new)
                p->finished_ids[p->n_finished++] = r.id;
        } else {
            const int i = p->n_chunks++;
            p->chunk_ids[i] = r.id;
            p->chunk_prior[i] = r.prefilled;
            p->chunk_len[i] = it.n;
            int rc = pkv_seqs_append(s->seqs, r.id, it.n, p->chunk_slots + p->n_chunk_tokens);
            if (rc != PKV_OK)
                return rc;
            p->n_chunk_tokens += it.n;
            r.prefilled += it.n;
            if (r.prefilled == r.prompt) {
                r.generated = 1;      // the prompt's last position yields the first token
                p->first_ids[p->n_first++] = r.id;
                if (r.generated >= r.max_new)
                    p->finished_ids[p->n_finished++] = r.id;
            }
        }
    }
    for (int64_t id : preempted)
        p->preempted_ids[p->n_preempted++] = id;

    // Finished sequences leave the running set now and release their blocks
    // at the next step.
    for (int i = 0; i < p->n_finished; ++i) {
        const int64_t id = p->finished_ids[i];
        s->running.erase(std::remove_if(s->running.begin(), s->running.end(),
                                        [&](const Req &r) { return r.id == id; }),
                         s->running.end());
        s->to_release.push_back(id);
    }
    return PKV_OK;
}
