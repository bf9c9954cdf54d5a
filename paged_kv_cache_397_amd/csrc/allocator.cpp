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
// Prefix caching (same section; ksqn.cn page, 3.4 and 5.2 item 4): a full block
// whose K/V are written can be offered to a cache keyed by a chain hash of its
// tokens and its predecessor's key, so that a later prompt opening with the same
// tokens takes those blocks instead of computing them again.  A cached block
// without holders stays in the free queue, findable, until an allocation takes
// it from the head (eviction).  Hits may leave the middle of the queue, so the
// queue is a doubly linked list over block IDs.
//
// Swapping (hihuo.com page, Preemption（抢占）: the Recompute and Swap modes;
// ksqn.cn page, 3.4 on --swap-space): a suspended sequence's blocks move to a
// host pool with its own FIFO queue and come back later onto fresh device blocks;
// the caller copies the data with pa_swap_blocks.
//
// Plain C++17, no HIP: this file also builds with g++ alone.

#include <cstdint>
#include <cstring>
#include <deque>
#include <new>
#include <unordered_map>
#include <vector>

#include "pagedkv.h"

namespace {

// FNV-1a, 64 bits, as published by its authors: xor each byte in, then multiply
// by the prime.
constexpr uint64_t kFnvOffset = 0xCBF29CE484222325ull;
constexpr uint64_t kFnvPrime = 0x100000001B3ull;

inline uint64_t fnv_byte(uint64_t h, uint8_t b) { return (h ^ b) * kFnvPrime; }

// Key of a full block: its parent's key (8 bytes, little-endian) followed by its
// tokens (4 bytes each, little-endian), hashed with FNV-1a-64.
uint64_t chain_hash(uint64_t parent, const int32_t* tokens, int32_t n) {
    uint64_t h = kFnvOffset;
    for (int k = 0; k < 8; ++k) h = fnv_byte(h, static_cast<uint8_t>(parent >> (8 * k)));
    for (int32_t i = 0; i < n; ++i) {
        const uint32_t t = static_cast<uint32_t>(tokens[i]);
        for (int k = 0; k < 4; ++k) h = fnv_byte(h, static_cast<uint8_t>(t >> (8 * k)));
    }
    return h;
}

}  // namespace

struct pa_allocator {
    struct Seq {
        std::vector<int32_t> table;
        int32_t len = 0;
        int32_t reg_done = 0;   // leading full blocks already offered to the prefix cache
        uint64_t reg_hash = 0;  // chain key after them
        bool swapped = false;   // table holds host blocks
    };
    int32_t num_blocks = 0;
    int32_t block_size = 0;
    // free queue (FIFO): a doubly linked list over block IDs, -1 terminated
    std::vector<int32_t> next, prev;
    std::vector<char> in_free;
    int32_t head = -1, tail = -1, nfree = 0;
    std::vector<int32_t> ref;
    std::unordered_map<int64_t, Seq> seqs;
    // prefix cache
    std::unordered_map<uint64_t, int32_t> cached;  // key -> block
    std::vector<uint64_t> key;                     // block -> key, when is_cached
    std::vector<char> is_cached;
    int64_t lookups = 0, hits = 0;
    // host pool for swapped sequences (FIFO)
    int32_t num_host_blocks = 0;
    std::deque<int32_t> host_free;

    // A resident (not swapped) sequence, or nullptr.
    Seq* resident(int64_t id) {
        auto it = seqs.find(id);
        return (it == seqs.end() || it->second.swapped) ? nullptr : &it->second;
    }
    const Seq* resident(int64_t id) const {
        auto it = seqs.find(id);
        return (it == seqs.end() || it->second.swapped) ? nullptr : &it->second;
    }

    void push_back(int32_t b) {
        prev[b] = tail;
        next[b] = -1;
        if (tail >= 0) next[tail] = b; else head = b;
        tail = b;
        in_free[b] = 1;
        ++nfree;
    }
    void unlink(int32_t b) {
        if (prev[b] >= 0) next[prev[b]] = next[b]; else head = next[b];
        if (next[b] >= 0) prev[next[b]] = prev[b]; else tail = prev[b];
        in_free[b] = 0;
        --nfree;
    }
    // The head of the free queue for a new use; a cached block is evicted.
    int32_t take() {
        const int32_t b = head;
        unlink(b);
        if (is_cached[b]) {
            cached.erase(key[b]);
            is_cached[b] = 0;
        }
        ref[b] = 1;
        return b;
    }
    void release_block(int32_t b) {
        if (--ref[b] == 0) push_back(b);
    }

    // Reserve the slot of seq's next token; see pa_seq_append.
    pa_status append(int64_t id, int64_t* slot, int32_t* cow_src, int32_t* cow_dst,
                     int32_t* new_block, int32_t* new_col) {
        Seq* sp = resident(id);
        if (!sp) return PA_ERR_STATE;
        Seq& s = *sp;
        const int32_t pos = s.len;
        const int32_t j = pos / block_size;
        int32_t src = -1, dst = -1, fresh = -1;
        if (j == static_cast<int32_t>(s.table.size())) {
            if (nfree == 0) return PA_ERR_OOM;
            fresh = take();
            s.table.push_back(fresh);
        } else if (ref[s.table[j]] > 1) {
            if (nfree == 0) return PA_ERR_OOM;
            fresh = take();
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
    a->next.assign(num_blocks, -1);
    a->prev.assign(num_blocks, -1);
    a->in_free.assign(num_blocks, 0);
    a->key.assign(num_blocks, 0);
    a->is_cached.assign(num_blocks, 0);
    if (initial_free_order) {
        for (int32_t k = 0; k < num_blocks; ++k) {
            const int32_t b = initial_free_order[k];
            if (b < 0 || b >= num_blocks || a->in_free[b]) {
                delete a;
                return PA_ERR_INVALID_ARG;
            }
            a->push_back(b);
        }
    } else {
        for (int32_t b = 0; b < num_blocks; ++b) a->push_back(b);
    }
    *out = a;
    return PA_OK;
}

void pa_alloc_destroy(pa_allocator* a) { delete a; }

int32_t pa_alloc_num_free(const pa_allocator* a) { return a ? a->nfree : -1; }

int32_t pa_alloc_num_seqs(const pa_allocator* a) {
    return a ? static_cast<int32_t>(a->seqs.size()) : -1;
}

int32_t pa_alloc_refcount(const pa_allocator* a, int32_t block) {
    if (!a || block < 0 || block >= a->num_blocks) return -1;
    return a->ref[block];
}

pa_status pa_alloc_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n) {
    if (!a || !n || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID_ARG;
    *n = a->nfree;
    int32_t k = 0;
    for (int32_t b = a->head; b >= 0 && k < cap; b = a->next[b]) out[k++] = b;
    return PA_OK;
}

pa_status pa_seq_add(pa_allocator* a, int64_t seq, int32_t num_tokens) {
    if (!a || num_tokens < 0) return PA_ERR_INVALID_ARG;
    if (a->seqs.count(seq)) return PA_ERR_STATE;
    const int64_t need = (static_cast<int64_t>(num_tokens) + a->block_size - 1) / a->block_size;
    if (need > a->nfree) return PA_ERR_OOM;
    pa_allocator::Seq s;
    s.table.reserve(static_cast<size_t>(need));
    for (int64_t k = 0; k < need; ++k) s.table.push_back(a->take());
    s.len = num_tokens;
    a->seqs.emplace(seq, std::move(s));
    return PA_OK;
}

pa_status pa_seq_add_prefix(pa_allocator* a, int64_t seq, const int32_t* tokens,
                            int32_t num_tokens, int32_t* num_cached_tokens) {
    if (!a || num_tokens < 0 || (num_tokens > 0 && !tokens)) return PA_ERR_INVALID_ARG;
    if (a->seqs.count(seq)) return PA_ERR_STATE;
    const int32_t B = a->block_size;
    const int32_t eligible = num_tokens > 0 ? (num_tokens - 1) / B : 0;  // never the last token's block
    std::vector<int32_t> hit;
    uint64_t h = 0;
    for (int32_t i = 0; i < eligible; ++i) {
        const uint64_t hi = chain_hash(h, tokens + static_cast<int64_t>(i) * B, B);
        auto it = a->cached.find(hi);
        if (it == a->cached.end()) break;
        hit.push_back(it->second);
        h = hi;
    }
    const int64_t total = (static_cast<int64_t>(num_tokens) + B - 1) / B;
    const int64_t need = total - static_cast<int64_t>(hit.size());
    int64_t idle = 0;
    for (int32_t b : hit) idle += a->ref[b] == 0;
    if (need > a->nfree - idle) return PA_ERR_OOM;
    a->lookups += eligible;
    a->hits += static_cast<int64_t>(hit.size());
    pa_allocator::Seq s;
    s.table.reserve(static_cast<size_t>(total));
    for (int32_t b : hit) {
        if (a->ref[b] == 0) a->unlink(b);
        a->ref[b] += 1;
        s.table.push_back(b);
    }
    for (int64_t k = 0; k < need; ++k) s.table.push_back(a->take());
    s.len = num_tokens;
    s.reg_done = static_cast<int32_t>(hit.size());
    s.reg_hash = h;
    a->seqs.emplace(seq, std::move(s));
    if (num_cached_tokens) *num_cached_tokens = static_cast<int32_t>(hit.size()) * B;
    return PA_OK;
}

pa_status pa_seq_register_blocks(pa_allocator* a, int64_t seq, const int32_t* tokens,
                                 int32_t num_tokens) {
    if (!a || num_tokens < 0 || (num_tokens > 0 && !tokens)) return PA_ERR_INVALID_ARG;
    pa_allocator::Seq* sp = a->resident(seq);
    if (!sp) return PA_ERR_STATE;
    pa_allocator::Seq& s = *sp;
    if (num_tokens > s.len) return PA_ERR_INVALID_ARG;
    const int32_t B = a->block_size;
    for (int32_t i = s.reg_done; i < num_tokens / B; ++i) {
        s.reg_hash = chain_hash(s.reg_hash, tokens + static_cast<int64_t>(i) * B, B);
        const int32_t b = s.table[i];
        if (!a->is_cached[b] && !a->cached.count(s.reg_hash)) {
            a->cached.emplace(s.reg_hash, b);
            a->key[b] = s.reg_hash;
            a->is_cached[b] = 1;
        }
        s.reg_done = i + 1;
    }
    return PA_OK;
}

pa_status pa_alloc_prefix_stats(const pa_allocator* a, int64_t* lookups, int64_t* hits,
                                int32_t* cached_blocks) {
    if (!a) return PA_ERR_INVALID_ARG;
    if (lookups) *lookups = a->lookups;
    if (hits) *hits = a->hits;
    if (cached_blocks) *cached_blocks = static_cast<int32_t>(a->cached.size());
    return PA_OK;
}

int32_t pa_alloc_block_cached(const pa_allocator* a, int32_t block, uint64_t* key) {
    if (!a || block < 0 || block >= a->num_blocks) return -1;
    if (!a->is_cached[block]) return 0;
    if (key) *key = a->key[block];
    return 1;
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
    const pa_allocator::Seq* p = a->resident(parent);
    if (!p || a->seqs.count(child)) return PA_ERR_STATE;
    pa_allocator::Seq c = *p;
    for (int32_t b : c.table) a->ref[b] += 1;
    a->seqs.emplace(child, std::move(c));
    return PA_OK;
}

pa_status pa_seq_free(pa_allocator* a, int64_t seq) {
    if (!a) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return PA_ERR_STATE;
    if (it->second.swapped) {
        for (int32_t h : it->second.table) a->host_free.push_back(h);
    } else {
        for (int32_t b : it->second.table) a->release_block(b);
    }
    a->seqs.erase(it);
    return PA_OK;
}

pa_status pa_seq_slots(const pa_allocator* a, int64_t seq, int32_t start, int32_t count,
                       int64_t* out) {
    if (!a || start < 0 || count < 0 || (count > 0 && !out)) return PA_ERR_INVALID_ARG;
    const pa_allocator::Seq* sp = a->resident(seq);
    if (!sp) return PA_ERR_STATE;
    const auto& s = *sp;
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
    const pa_allocator::Seq* sp = a->resident(seq);
    if (!sp) return PA_ERR_STATE;
    const auto& t = sp->table;
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
        const pa_allocator::Seq* sp = a->resident(seqs[k]);
        if (!sp) return PA_ERR_STATE;
        if (static_cast<int64_t>(sp->table.size()) > max_blocks_per_seq) return PA_ERR_INVALID_ARG;
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

pa_status pa_alloc_set_host_pool(pa_allocator* a, int32_t num_host_blocks) {
    if (!a || num_host_blocks < 0) return PA_ERR_INVALID_ARG;
    for (const auto& kv : a->seqs)
        if (kv.second.swapped) return PA_ERR_STATE;
    a->num_host_blocks = num_host_blocks;
    a->host_free.clear();
    for (int32_t h = 0; h < num_host_blocks; ++h) a->host_free.push_back(h);
    return PA_OK;
}

pa_status pa_alloc_host_free_list(const pa_allocator* a, int32_t* out, int32_t cap, int32_t* n) {
    if (!a || !n || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID_ARG;
    *n = static_cast<int32_t>(a->host_free.size());
    int32_t k = 0;
    for (auto it = a->host_free.begin(); it != a->host_free.end() && k < cap; ++it) out[k++] = *it;
    return PA_OK;
}

pa_status pa_seq_host_blocks(const pa_allocator* a, int64_t seq, int32_t* out, int32_t cap) {
    if (!a || cap < 0 || (cap > 0 && !out)) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end() || !it->second.swapped) return PA_ERR_STATE;
    const auto& t = it->second.table;
    if (static_cast<int64_t>(t.size()) > cap) return PA_ERR_INVALID_ARG;
    if (!t.empty()) std::memcpy(out, t.data(), t.size() * sizeof(int32_t));
    return PA_OK;
}

int32_t pa_alloc_num_free_host(const pa_allocator* a) {
    return a ? static_cast<int32_t>(a->host_free.size()) : -1;
}

int32_t pa_seq_is_swapped(const pa_allocator* a, int64_t seq) {
    if (!a) return -1;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end()) return -1;
    return it->second.swapped ? 1 : 0;
}

pa_status pa_seq_swap_out(pa_allocator* a, int64_t seq, int32_t* pairs, int32_t cap,
                          int32_t* num_pairs) {
    if (!a || cap < 0 || (cap > 0 && !pairs) || !num_pairs) return PA_ERR_INVALID_ARG;
    pa_allocator::Seq* sp = a->resident(seq);
    if (!sp) return PA_ERR_STATE;
    const int32_t n = static_cast<int32_t>(sp->table.size());
    if (n > cap) return PA_ERR_INVALID_ARG;
    if (n > static_cast<int32_t>(a->host_free.size())) return PA_ERR_OOM;
    for (int32_t k = 0; k < n; ++k) {
        const int32_t b = sp->table[k];
        const int32_t h = a->host_free.front();
        a->host_free.pop_front();
        pairs[2 * k] = b;
        pairs[2 * k + 1] = h;
        sp->table[k] = h;
        a->release_block(b);
    }
    sp->swapped = true;
    *num_pairs = n;
    return PA_OK;
}

pa_status pa_seq_swap_in(pa_allocator* a, int64_t seq, int32_t* pairs, int32_t cap,
                         int32_t* num_pairs) {
    if (!a || cap < 0 || (cap > 0 && !pairs) || !num_pairs) return PA_ERR_INVALID_ARG;
    auto it = a->seqs.find(seq);
    if (it == a->seqs.end() || !it->second.swapped) return PA_ERR_STATE;
    pa_allocator::Seq& s = it->second;
    const int32_t n = static_cast<int32_t>(s.table.size());
    if (n > cap) return PA_ERR_INVALID_ARG;
    if (n > a->nfree) return PA_ERR_OOM;
    for (int32_t k = 0; k < n; ++k) {
        const int32_t h = s.table[k];
        const int32_t b = a->take();
        pairs[2 * k] = h;
        pairs[2 * k + 1] = b;
        s.table[k] = b;
        a->host_free.push_back(h);
    }
    s.swapped = false;
    *num_pairs = n;
    return PA_OK;
}

}  // extern "C"
