// Continuous-batching scheduler behind the pa_sched_* entry points: the host side
// of a serving loop over the block allocator (hihuo.com "vLLM 原理：PagedAttention 和
// Continuous Batching", vLLM 的调度 > 调度流程 and Preemption（抢占）; ksqn.cn
// "大模型推理性能优化：PagedAttention与Continuous Batching原理与实践", section 2.3).
// The step order is stated in include/pagedkv.h.  Every block operation goes
// through the allocator's C entry points, so the scheduler holds no block state
// of its own: only requests, queues and the last step's plan.
//
// Plain C++17, no HIP: this file also builds with g++ alone.

#include <cstdint>
#include <deque>
#include <memory>
#include <new>
#include <vector>

#include "pagedkv.h"

namespace {

struct Req {
    int64_t rid = 0;
    int32_t prompt = 0;      // prompt tokens as submitted
    int32_t out_len = 0;     // tokens to generate
    int32_t generated = 0;   // tokens generated so far (decode appends)
    int32_t prompt_eff = 0;  // tokens to prefill at (re)admission: prompt + generated
    int32_t prefilled = 0;   // prompt tokens whose chunk has been planned
    int32_t length = 0;      // tokens held in the cache
    bool ready = false;      // prompt complete before this step: decodes
    enum State { Pending, Waiting, Running, Swapped } state = Pending;
    std::vector<int32_t> known;  // prefix caching: prompt + known output token IDs
};

}  // namespace

struct pa_scheduler {
    pa_allocator* alloc = nullptr;
    int32_t block_size = 0;
    int32_t chunk = 0;
    bool prefix = false;
    bool swap = false;
    int64_t steps = 0;
    std::vector<std::unique_ptr<Req>> reqs;  // by rid; reset when a request ends
    std::vector<Req*> pending;               // added since the last step
    std::deque<Req*> waiting, swapped_q;
    std::vector<Req*> running;

    // the last step's plan
    std::vector<int64_t> finished, arrived, admitted, preempted, prefill_rid, prefill_slots;
    std::vector<int32_t> admitted_cached, prefill_start, prefill_count;
    std::vector<int64_t> decode_rid, decode_pos, decode_slot;
    std::vector<int32_t> decode_cow;
    std::vector<int64_t> swapped_in, swapped_out;
    std::vector<int32_t> swapped_in_pairs, swapped_out_pairs, swap_in, swap_out;
    // scratch
    std::vector<int64_t> ids, slots;
    std::vector<int32_t> cows, pairs;
    std::vector<Req*> batch;

    ~pa_scheduler() { pa_alloc_destroy(alloc); }

    void clear_plan() {
        finished.clear(); arrived.clear(); admitted.clear(); admitted_cached.clear();
        preempted.clear(); prefill_rid.clear(); prefill_start.clear(); prefill_count.clear();
        prefill_slots.clear(); decode_rid.clear(); decode_pos.clear(); decode_slot.clear();
        decode_cow.clear(); swapped_in.clear(); swapped_out.clear(); swapped_in_pairs.clear();
        swapped_out_pairs.clear(); swap_in.clear(); swap_out.clear();
    }

    // Move a sequence's blocks between the device and the host pool; appends the
    // pairs to `out` and returns the allocator's status.
    pa_status swap_call(bool in, int64_t rid, std::vector<int32_t>& out, int32_t* n) {
        int32_t nt = 0, nb = 0;
        pa_status st = pa_seq_info(alloc, rid, &nt, &nb);
        if (st != PA_OK) return st;
        pairs.resize(2 * static_cast<size_t>(nb > 0 ? nb : 1));
        st = in ? pa_seq_swap_in(alloc, rid, pairs.data(), nb, n)
                : pa_seq_swap_out(alloc, rid, pairs.data(), nb, n);
        if (st == PA_OK) out.insert(out.end(), pairs.begin(), pairs.begin() + 2 * *n);
        return st;
    }

    pa_status step();
};

pa_status pa_scheduler::step() {
    const int32_t B = block_size;
    // Every decode token's ID must be known before anything changes (prefix caching).
    if (prefix) {
        for (Req* r : running)
            if (r->ready && r->generated < r->out_len &&
                static_cast<int64_t>(r->known.size()) <= r->prompt + r->generated)
                return PA_ERR_STATE;
        for (Req* r : swapped_q)
            if (r->ready && r->generated < r->out_len &&
                static_cast<int64_t>(r->known.size()) <= r->prompt + r->generated)
                return PA_ERR_STATE;
    }
    clear_plan();
    // 1. finished requests release their blocks
    {
        size_t k = 0;
        for (Req* r : running) {
            if (r->generated >= r->out_len) {
                const pa_status st = pa_seq_free(alloc, r->rid);
                if (st != PA_OK) return st;
                finished.push_back(r->rid);
                reqs[static_cast<size_t>(r->rid)].reset();
            } else {
                running[k++] = r;
            }
        }
        running.resize(k);
    }
    // 2. arrivals
    for (Req* r : pending) {
        r->state = Req::Waiting;
        waiting.push_back(r);
        arrived.push_back(r->rid);
    }
    pending.clear();
    // 3. swapped requests come back first
    while (!swapped_q.empty()) {
        Req* r = swapped_q.front();
        int32_t n = 0;
        const pa_status st = swap_call(true, r->rid, swap_in, &n);
        if (st == PA_ERR_OOM) break;
        if (st != PA_OK) return st;
        swapped_q.pop_front();
        r->state = Req::Running;
        running.push_back(r);
        swapped_in.push_back(r->rid);
        swapped_in_pairs.push_back(n);
    }
    // 4. admissions, first come first served
    while (!waiting.empty() && swapped_q.empty()) {
        Req* r = waiting.front();
        int32_t cached = 0;
        if (prefix) {
            const pa_status st =
                pa_seq_add_prefix(alloc, r->rid, r->known.data(), r->prompt_eff, &cached);
            if (st == PA_ERR_OOM) break;
            if (st != PA_OK) return st;
        } else {
            if ((static_cast<int64_t>(r->prompt_eff) + B - 1) / B > pa_alloc_num_free(alloc)) break;
            const pa_status st = pa_seq_add(alloc, r->rid, r->prompt_eff);
            if (st != PA_OK) return st;
        }
        r->length = r->prompt_eff;
        r->prefilled = cached;
        r->ready = false;
        r->state = Req::Running;
        running.push_back(r);
        waiting.pop_front();
        admitted.push_back(r->rid);
        admitted_cached.push_back(cached);
    }
    // 5. decode appends; out of blocks: preempt the running request admitted last
    batch.clear();
    for (Req* r : running)
        if (r->ready) batch.push_back(r);
    size_t from = 0;
    while (from < batch.size()) {
        const int32_t n = static_cast<int32_t>(batch.size() - from);
        ids.resize(static_cast<size_t>(n));
        slots.resize(static_cast<size_t>(n));
        cows.resize(2 * static_cast<size_t>(n));
        for (int32_t k = 0; k < n; ++k) ids[static_cast<size_t>(k)] = batch[from + static_cast<size_t>(k)]->rid;
        int32_t done = 0;
        const pa_status st = pa_seq_append_batch(alloc, ids.data(), n, slots.data(), cows.data(),
                                                 nullptr, nullptr, &done);
        for (int32_t k = 0; k < done; ++k) {
            Req* r = batch[from + static_cast<size_t>(k)];
            decode_rid.push_back(r->rid);
            decode_pos.push_back(r->length);
            decode_slot.push_back(slots[static_cast<size_t>(k)]);
            decode_cow.push_back(cows[2 * static_cast<size_t>(k)]);
            decode_cow.push_back(cows[2 * static_cast<size_t>(k) + 1]);
            r->length += 1;
            r->generated += 1;
        }
        from += static_cast<size_t>(done);
        if (st == PA_OK) break;
        if (st != PA_ERR_OOM) return st;
        Req* victim = running.back();
        running.pop_back();
        int32_t nt = 0, nb = 0;
        pa_status sv = pa_seq_info(alloc, victim->rid, &nt, &nb);
        if (sv != PA_OK) return sv;
        if (swap && nb <= pa_alloc_num_free_host(alloc)) {
            int32_t np = 0;
            sv = swap_call(false, victim->rid, swap_out, &np);
            if (sv != PA_OK) return sv;
            victim->state = Req::Swapped;
            swapped_q.push_back(victim);
            swapped_out.push_back(victim->rid);
            swapped_out_pairs.push_back(np);
        } else {
            sv = pa_seq_free(alloc, victim->rid);
            if (sv != PA_OK) return sv;
            victim->prompt_eff = victim->prompt + victim->generated;
            victim->prefilled = 0;
            victim->ready = false;
            victim->state = Req::Waiting;
            waiting.push_front(victim);
            preempted.push_back(victim->rid);
        }
        // the victim, if it was still to append, no longer does
        size_t k = from;
        for (size_t i = from; i < batch.size(); ++i)
            if (batch[i] != victim) batch[k++] = batch[i];
        batch.resize(k);
    }
    // 6. prompt chunks, after the appends
    for (Req* r : running) {
        if (r->prefilled >= r->prompt_eff) continue;
        const int32_t c = r->prompt_eff - r->prefilled < chunk ? r->prompt_eff - r->prefilled : chunk;
        const size_t at = prefill_slots.size();
        prefill_slots.resize(at + static_cast<size_t>(c));
        const pa_status st = pa_seq_slots(alloc, r->rid, r->prefilled, c, prefill_slots.data() + at);
        if (st != PA_OK) return st;
        prefill_rid.push_back(r->rid);
        prefill_start.push_back(r->prefilled);
        prefill_count.push_back(c);
        r->prefilled += c;
        if (prefix) {
            const pa_status sr = pa_seq_register_blocks(alloc, r->rid, r->known.data(), r->prefilled);
            if (sr != PA_OK) return sr;
        }
    }
    // 7. a decode token that completes a block offers it to the prefix cache
    if (prefix) {
        for (size_t k = 0; k < decode_rid.size(); ++k) {
            if ((decode_pos[k] + 1) % B != 0) continue;
            Req* r = reqs[static_cast<size_t>(decode_rid[k])].get();
            if (!r || r->state != Req::Running) continue;
            const pa_status st =
                pa_seq_register_blocks(alloc, r->rid, r->known.data(), r->prompt + r->generated);
            if (st != PA_OK) return st;
        }
    }
    for (Req* r : running)
        if (!r->ready && r->prefilled == r->prompt_eff) r->ready = true;
    return PA_OK;
}

extern "C" {

pa_status pa_sched_create(int32_t num_blocks, int32_t block_size,
                          const int32_t* initial_free_order, int32_t chunk,
                          int32_t prefix_caching, int32_t num_host_blocks, pa_scheduler** out) {
    if (!out || chunk <= 0 || num_host_blocks < 0) return PA_ERR_INVALID_ARG;
    *out = nullptr;
    pa_scheduler* s = new (std::nothrow) pa_scheduler();
    if (!s) return PA_ERR_OOM;
    pa_status st = pa_alloc_create(num_blocks, block_size, initial_free_order, &s->alloc);
    if (st == PA_OK && num_host_blocks > 0) st = pa_alloc_set_host_pool(s->alloc, num_host_blocks);
    if (st != PA_OK) {
        delete s;
        return st;
    }
    s->block_size = block_size;
    s->chunk = chunk;
    s->prefix = prefix_caching != 0;
    s->swap = num_host_blocks > 0;
    *out = s;
    return PA_OK;
}

void pa_sched_destroy(pa_scheduler* s) { delete s; }

pa_allocator* pa_sched_allocator(pa_scheduler* s) { return s ? s->alloc : nullptr; }

pa_status pa_sched_add_requests(pa_scheduler* s, int32_t n, const int32_t* prompt_lens,
                                const int32_t* out_lens, const int32_t* prompt_tokens,
                                const int32_t* out_tokens, int64_t* rids) {
    if (!s || n < 0 || (n > 0 && (!prompt_lens || !out_lens))) return PA_ERR_INVALID_ARG;
    if (n > 0 && s->prefix && !prompt_tokens) return PA_ERR_INVALID_ARG;
    for (int32_t k = 0; k < n; ++k)
        if (prompt_lens[k] < 0 || out_lens[k] < 0) return PA_ERR_INVALID_ARG;
    const size_t base = s->reqs.size();
    // all or nothing: every request is built before any is queued
    std::vector<std::unique_ptr<Req>> made;
    made.reserve(static_cast<size_t>(n));
    int64_t pt = 0, ot = 0;
    for (int32_t k = 0; k < n; ++k) {
        std::unique_ptr<Req> r(new (std::nothrow) Req());
        if (!r) return PA_ERR_OOM;
        r->rid = static_cast<int64_t>(base) + k;
        r->prompt = prompt_lens[k];
        r->out_len = out_lens[k];
        r->prompt_eff = r->prompt;
        if (s->prefix) {
            r->known.assign(prompt_tokens + pt, prompt_tokens + pt + prompt_lens[k]);
            if (out_tokens) r->known.insert(r->known.end(), out_tokens + ot, out_tokens + ot + out_lens[k]);
        }
        pt += prompt_lens[k];
        ot += out_lens[k];
        made.push_back(std::move(r));
    }
    for (int32_t k = 0; k < n; ++k) {
        if (rids) rids[k] = made[static_cast<size_t>(k)]->rid;
        s->pending.push_back(made[static_cast<size_t>(k)].get());
        s->reqs.push_back(std::move(made[static_cast<size_t>(k)]));
    }
    return PA_OK;
}

pa_status pa_sched_push_tokens(pa_scheduler* s, const int64_t* rids, const int32_t* tokens,
                               int32_t n) {
    if (!s || n < 0 || (n > 0 && (!rids || !tokens))) return PA_ERR_INVALID_ARG;
    for (int32_t k = 0; k < n; ++k)
        if (rids[k] < 0 || rids[k] >= static_cast<int64_t>(s->reqs.size()) ||
            !s->reqs[static_cast<size_t>(rids[k])])
            return PA_ERR_STATE;
    for (int32_t k = 0; k < n; ++k) s->reqs[static_cast<size_t>(rids[k])]->known.push_back(tokens[k]);
    return PA_OK;
}

pa_status pa_sched_step(pa_scheduler* s, pa_sched_plan* p) {
    if (!s || !p) return PA_ERR_INVALID_ARG;
    const pa_status st = s->step();
    if (st != PA_OK) return st;
    p->step = s->steps++;
    p->num_finished = static_cast<int32_t>(s->finished.size());
    p->num_arrived = static_cast<int32_t>(s->arrived.size());
    p->num_admitted = static_cast<int32_t>(s->admitted.size());
    p->num_preempted = static_cast<int32_t>(s->preempted.size());
    p->num_prefill = static_cast<int32_t>(s->prefill_rid.size());
    p->num_decode = static_cast<int32_t>(s->decode_rid.size());
    int32_t nc = 0;
    for (size_t k = 0; k < s->decode_rid.size(); ++k) nc += s->decode_cow[2 * k] >= 0;
    p->num_decode_cows = nc;
    p->num_swapped_in = static_cast<int32_t>(s->swapped_in.size());
    p->num_swapped_out = static_cast<int32_t>(s->swapped_out.size());
    p->num_prefill_tokens = static_cast<int64_t>(s->prefill_slots.size());
    p->finished = s->finished.data();
    p->arrived = s->arrived.data();
    p->admitted = s->admitted.data();
    p->admitted_cached = s->admitted_cached.data();
    p->preempted = s->preempted.data();
    p->prefill_rid = s->prefill_rid.data();
    p->prefill_start = s->prefill_start.data();
    p->prefill_count = s->prefill_count.data();
    p->prefill_slots = s->prefill_slots.data();
    p->decode_rid = s->decode_rid.data();
    p->decode_pos = s->decode_pos.data();
    p->decode_slot = s->decode_slot.data();
    p->decode_cow = s->decode_cow.data();
    p->swapped_in = s->swapped_in.data();
    p->swapped_in_pairs = s->swapped_in_pairs.data();
    p->swap_in = s->swap_in.data();
    p->swapped_out = s->swapped_out.data();
    p->swapped_out_pairs = s->swapped_out_pairs.data();
    p->swap_out = s->swap_out.data();
    return PA_OK;
}

int32_t pa_sched_running(const pa_scheduler* s, int64_t* rids, int32_t* prompts, int32_t* lengths,
                         int32_t cap) {
    if (!s || cap < 0) return -1;
    const int32_t n = static_cast<int32_t>(s->running.size());
    for (int32_t k = 0; k < n && k < cap; ++k) {
        const Req* r = s->running[static_cast<size_t>(k)];
        if (rids) rids[k] = r->rid;
        if (prompts) prompts[k] = r->prompt;
        if (lengths) lengths[k] = r->length;
    }
    return n;
}

int32_t pa_sched_waiting(const pa_scheduler* s, int64_t* rids, int32_t cap) {
    if (!s || cap < 0) return -1;
    const int32_t n = static_cast<int32_t>(s->waiting.size());
    int32_t k = 0;
    for (auto it = s->waiting.begin(); it != s->waiting.end() && k < cap; ++it) {
        if (rids) rids[k] = (*it)->rid;
        ++k;
    }
    return n;
}

}  // extern "C"
