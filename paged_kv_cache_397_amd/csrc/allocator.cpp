// Host block allocator behind the pa_alloc_* / pa_seq_* entry points.
//
// Block manager of the paged KV cache: fixed-size pages drawn from a free
// list with no contiguous search (ksqn.cn "大模型推理性能优化：PagedAttention与
// Continuous Batching原理与实践", section 2.2), per-request page tables grown
// on demand and released at once when a request ends (hihuo.com "vLLM 原理：
// PagedAttention 和 Continuous Batching", PagedAttention > 工作原理 1-3), a FIFO
// pool of block IDs allocated ceil(n / B) at a time (blog.gitcode.com
// "如何通过PagedAttention实现LLM高性能推理：实战指南", section 2.2), and pages
// shared between sequences (hihuo.com page, 优势 > 3. 支持共享) with reference
// counts and copy-on-write.  Every operation either succeeds or leaves the
// state untouched.
//
// Plain C++17, no HIP: this file also builds with g++ alone.

#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

struct pa_allocator {
    struct Seq {
        std::vector<int32_t> table;
        int32_t len = 0;
    };
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    std::deque<int32_t> free_q;
    std::vector<int32_t> ref;
    std::unordered_map<int64_t, Seq> seqs;

    // Reserve the slot of seq's next token; see pa_seq_append.
    pa_status append(int64_t id, int64_t* slot, int32_t* cow_src, int32_t* cow_dst,
                     int32_t* new_block, int32_t* new_col) {
        auto it = seqs.find(id);
        if (it == seqs.end()) return PA_ERR_STATE;
        Seq& s = it->second;
        const int32_t pos = s.len;
        const int32_t j = pos / block_size;
        int32_t src = -1, dst = -1, fresh = -1;
        if (j == static_cast<int32_t>(s.table.size())) {
            if (free_q.empty()) return PA_ERR_OOM;
            fresh = free_q.front();
            free_q.pop_front();
            ref[fresh] = 1;
            s.table.push_back(fresh);
        } else if (ref[s.table[j]] > 1) {
            if (free_q.empty()) return PA_ERR_OOM;
            fresh = free_q.front();
            free_q.pop_front();
            ref[fresh] = 1;
            src = s.table[j];
            dst = fresh;
            ref[src] -= 1;
            s.table[j] = fresh;
        }
        s.len = pos + 1;
        if (slot) *slot = static_cast<int64_t>(s.table[j]) * block_size + pos % block_size;
        if (cow_src) *cow_src = src;
        if (cow_dst) *cow_dst = dst;
        if (new_block) *new_block = fresh;
        if (new_col) *new_col = fresh >= 0 ? j : -1;
        return PA_OK;
    }
};

extern "C" {

pa_status pa_alloc_create(int32_t num_blocks, int32_t block_size,
                          const int32_t* initial_free_order, pa_allocator** out) {
    if (!out || num_blocks <= 0 || block_size <= 0) return PA_ERR_INVALID_ARG;
    *out = nullptr;
    pa_allocator* a = new (std::nothrow) pa_allocator();
    if (!a) return PA_ERR_OOM;
    a->num_blocks = num_blocks;
    a->block_size = block_size;
    a->ref.assign(num_blocks, 0);
    if (initial_free_order) {
        std::vector<char> seen(num_blocks, 0);
        for (int32_t k = 0; k < num_blocks; ++k) {
            const int32_t b = initial_free_order[k];
            if (b < 0 || b >= num_blocks || seen[b]) {
                delete a;
                return PA_ERR_INVALID_ARG;
            }
            seen[b] = 1;
            a->free_q.push_back(b);
        }
    } else {
        for (int32_t b = 0; b < num_blocks; ++b) a->free_q.push_back(b);
    }
    *out = a;
    return PA_OK;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int32_t pa_alloc_num_free(const pa_allocator* a) {
    return a ? static_cast<int32_t>(a->free_q.size()) : -1;
}

int32_t pa_alloc_num_seqs(const pa_allocator* a) {
    return a ? static_cast<int32_t>(a->seqs.size()) : -1;
}

int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block) {
    if (!a || block < 0 || block >= a->num_blocks) return -1;
    return a->ref[block];
}

pa_status pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n) {
    if (!a || !n || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID_ARG;
    const int32_t len = static_cast<int32_t>(a->free_q.size());
    *n = len;
    int32_t k = 0;
    for (auto it = a->free_q.begin(); it != a->free_q.end() && k < cap; ++it) out[k++] = *it;
    return PA_OK;
}

pa_status pa_seq_add(pa_allocator* a, int64_t seq, int32_t num_tokens) {
    if (!a || num_tokens < 0) return PA_ERR_INVALID_ARG;
    if (a->seqs.count(seq)) return PA_ERR_STATE;
    const int64_t need = (static_cast<int64_t>(num_tokens) + a->block_size - 1) / a->block_size;
    if (need > static_cast<int64_t>(a->free_q.size())) return PA_ERR_OOM;
    pa_allocator::Seq s;
    s.table.reserve(static_cast<size_t>(need));
    for (int64_t k = 0; k < need; ++k) {
        const int32_t b = a->free_q.front();
        a->free_q.pop_front();
        a->ref[b] = 1;
        s.table.push_back(b);
    }
    s.len = num_tokens;
    a->seqs.emplace(seq, std::move(s));
    return PA_OK;
}

pa_status pa_seq_append(pa_allocator* a, int64_t seq, int64_t* slot, int32_t* cow_src,
                        int32_t* cow_dst) {
    if (!a) return PA_ERR_INVALID_ARG;
    return a->append(seq, slot, cow_src, cow_dst, nullptr, nullptr);
}

pa_status pa_seq_append_batch(pa_allocator* a, const int64_t* seqs, int32_t n, int64_t* slots,
                              int32_t* cow_pairs, int32_t* new_blocks, int32_t* new_cols,
                              int32_t* num_done) {
    if (!a || n < 0 || (n > 0 && (!seqs || !slots || !cow_pairs)) || !num_done)
        return PA_ERR_INVALID_ARG;
    *num_done = 0;
    for (int32_t k = 0; k < n; ++k) {
        const pa_status st = a->append(seqs[k], &slots[k], &cow_pairs[2 * k], &cow_pairs[2 * k + 1],
                                       new_blocks ? &new_blocks[k] : nullptr,
                                       new_cols ? &new_cols[k] : nullptr);
        if (st != PA_OK) return st;
        *num_done = k + 1;
    }
    return PA_OK;
}

pa_status pa_seq_fork(pa_allocator* a, int64_t parent, int64_t child) {
    if (!a) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(parent);
    if (it == a->seqs.end() || a->seqs.count(child)) return PA_ERR_STATE;
    pa_allocator::Seq c = it->second;
    for (int32_t b : c.table) a->ref[b] += 1;
    a->seqs.emplace(child, std::move(c));
    return PA_OK;
}

pa_status pa_seq_free(pa_allocator* a, int64_t seq) {
    if (!a) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return PA_ERR_STATE;
    for (int32_t b : it->second.table) {
        if (--a->ref[b] == 0) a->free_q.push_back(b);
    }
    a->seqs.erase(it);
    return PA_OK;
}

pa_status pa_seq_slots(const pa_allocator* a, int64_t seq, int32_t start, int32_t count,
                       int64_t* out) {
    if (!a || start < 0 || count < 0 || (count > 0 && !out)) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return PA_ERR_STATE;
    const auto& s = it->second;
    if (static_cast<int64_t>(start) + count > s.len) return PA_ERR_INVALID_ARG;
    const int32_t B = a->block_size;
    for (int32_t k = 0; k < count; ++k) {
        const int32_t p = start + k;
        out[k] = static_cast<int64_t>(s.table[p / B]) * B + p % B;
    }
    return PA_OK;
}

pa_status pa_seq_info(const pa_allocator* a, int64_t seq, int32_t* num_tokens,
                      int32_t* num_blocks) {
    if (!a) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return PA_ERR_STATE;
    if (num_tokens) *num_tokens = it->second.len;
    if (num_blocks) *num_blocks = static_cast<int32_t>(it->second.table.size());
    return PA_OK;
}

pa_status pa_seq_block_table(const pa_allocator* a, int64_t seq, int32_t* out, int32_t cap) {
    if (!a || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return PA_ERR_STATE;
    const auto& t = it->second.table;
    if (static_cast<int64_t>(t.size()) > cap) return PA_ERR_INVALID_ARG;
    if (!t.empty()) std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
    return PA_OK;
}

pa_status pa_batch_metadata(const pa_allocator* a, const int64_t* seqs, int32_t n,
                            int32_t max_blocks_per_seq, int32_t* block_tables,
                            int32_t* context_lens) {
    if (!a || n < 0 || max_blocks_per_seq < 0 ||
        (n > 0 && (!seqs || !context_lens || (max_blocks_per_seq > 0 && !block_tables))))
        return PA_ERR_INVALID_ARG;
    for (int32_t k = 0; k < n; ++k) {
        auto it = a->seqs.find(seqs[k]);
        if (it == a->seqs.end()) return PA_ERR_STATE;
        if (static_cast<int64_t>(it->second.table.size()) > max_blocks_per_seq)
            return PA_ERR_INVALID_ARG;
    }
    for (int32_t k = 0; k < n; ++k) {
        const auto& s = a->seqs.find(seqs[k])->second;
        int32_t* row = block_tables + static_cast<int64_t>(k) * max_blocks_per_seq;
        const int32_t nb = static_cast<int32_t>(s.table.size());
        if (nb) std::memcpy(row, s.table.data(), nb * sizeof(int32_t));
        for (int32_t c = nb; c < max_blocks_per_seq; ++c) row[c] = -1;
        context_lens[k] = s.len;
    }
    return PA_OK;
}

}  // extern "C"
