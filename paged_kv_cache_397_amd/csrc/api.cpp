// C ABI of libpagedkv: argument validation and kernel launches.  The kernels
// live in kernels_cache.hip, kernels_decode.hip and kernels_prefill.hip; the host
// allocator in allocator.cpp.  No entry point allocates device memory.

#include <atomic>
#include <cmath>
#include <cstdint>
#include <mutex>

#include "pagedkv.h"
#include "pagedkv_internal.h"

namespace {

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Checks a descriptor: INVALID_ARG for impossible values, UNSUPPORTED for
// valid ones this build has no kernels for.
pa_status check_desc(const pa_cache_desc* d) {
    if (!d) return PA_ERR_INVALID_ARG;
    if (d->num_blocks <= 0 || d->block_size <= 0 || d->num_kv_heads <= 0 || d->head_dim <= 0)
        return PA_ERR_INVALID_ARG;
    if (d->dtype != PA_DTYPE_F32 && d->dtype != PA_DTYPE_BF16) return PA_ERR_INVALID_ARG;
    if (d->block_size != 8 && d->block_size != 16 && d->block_size != 32 && d->block_size != 64)
        return PA_ERR_UNSUPPORTED;
    if (d->head_dim != 64 && d->head_dim != 128) return PA_ERR_UNSUPPORTED;
    return PA_OK;
}

size_t elem_bytes(const pa_cache_desc* d) { return d->dtype == PA_DTYPE_F32 ? 4 : 2; }

pa_status from_hip(hipError_t e) {
    if (e == hipSuccess) return PA_OK;
    if (e == hipErrorInvalidValue) {
        (void)hipGetLastError();
        return PA_ERR_UNSUPPORTED;
    }
    return PA_ERR_HIP;
}

bool group_kernel_for(const pa_cache_desc* d, int32_t group) {
    return d->dtype == PA_DTYPE_BF16 && group > 1;
}

// Workspace of W units: partial records (two per unit) | unit records, from the
// start; W split counts, from the end (count i is the i-th int32 before the end), so
// that calls with different unit counts on one workspace never write each other's
// counts.
// A decode step (pa_decode_step) also keeps, after the unit records, a 16-byte
// sync word block and 16 bytes of metadata per sequence.
struct WorkspaceLayout {
    size_t piece_floats;  // floats of one partial record
    size_t rec_offset;    // bytes to the unit records
    size_t step_offset;   // bytes to the decode step's sync words, then its per-sequence metadata
    size_t bytes;         // total
};

WorkspaceLayout workspace_layout(const pa_cache_desc* d, int32_t num_q_heads, int32_t units,
                                 int32_t step_seqs = -1) {
    const int32_t group = num_q_heads / d->num_kv_heads;
    const int32_t gh = group_kernel_for(d, group) ? group : 1;
    WorkspaceLayout w;
    w.piece_floats = static_cast<size_t>(gh) * d->head_dim + ((2 * gh + 3) & ~3);
    const size_t pieces = static_cast<size_t>(units) * 2 * w.piece_floats * sizeof(float);
    w.rec_offset = (pieces + 255) & ~size_t(255);
    const size_t recs = static_cast<size_t>(units) * pkv::kRecInts * sizeof(int32_t);
    w.step_offset = (w.rec_offset + recs + 15) & ~size_t(15);
    const size_t step = step_seqs < 0 ? 0 : 16 + static_cast<size_t>(step_seqs) * 16;
    w.bytes = (step_seqs < 0 ? w.rec_offset + recs : w.step_offset + step) +
              static_cast<size_t>(units) * sizeof(int32_t);
    return w;
}

size_t workspace_for(const pa_cache_desc* d, int32_t num_q_heads, int32_t units) {
    return workspace_layout(d, num_q_heads, units).bytes;
}

std::atomic<int32_t> g_default_units{0};

constexpr int32_t kMaxUnits = 1 << 20;

}  // namespace

extern "C" {

const char* pa_status_string(pa_status s) {
    switch (s) {
        case PA_OK: return "ok";
        case PA_ERR_INVALID_ARG: return "invalid argument";
        case PA_ERR_UNSUPPORTED: return "unsupported shape or dtype";
        case PA_ERR_OOM: return "out of free blocks";
        case PA_ERR_STATE: return "unknown, duplicate or already-freed sequence";
        case PA_ERR_HIP: return "HIP runtime error";
        case PA_ERR_TOO_LARGE: return "request needs more than the library's static scratch buffer holds";
    }
    return "unknown status";
}

int32_t pa_abi_version(void) { return (1 << 16) | 1; }

size_t pa_cache_bytes(const pa_cache_desc* d) {
    if (check_desc(d) != PA_OK) return 0;
    return static_cast<size_t>(d->num_blocks) * d->num_kv_heads * d->block_size * d->head_dim *
           elem_bytes(d);
}

pa_status pa_reshape_and_cache(const pa_cache_desc* d, const void* k, const void* v,
                               const int64_t* slot_mapping, int32_t num_tokens, void* k_cache,
                               void* v_cache, void* stream) {
    pa_status st = check_desc(d);
    if (st != PA_OK) return st;
    if (num_tokens < 0) return PA_ERR_INVALID_ARG;
    if (num_tokens == 0) return PA_OK;
    if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
    if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(slot_mapping, 8))
        return PA_ERR_INVALID_ARG;
    if (d->num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
    return from_hip(pkv::launch_reshape_and_cache(d->dtype, d->head_dim, d->block_size,
                                                  d->num_kv_heads, d->num_blocks, k, v,
                                                  slot_mapping, num_tokens, k_cache, v_cache,
                                                  static_cast<hipStream_t>(stream)));
}

pa_status pa_copy_blocks(const pa_cache_desc* d, void* k_cache, void* v_cache,
                         const int32_t* pairs, int32_t num_pairs, void* stream) {
    pa_status st = check_desc(d);
    if (st != PA_OK) return st;
    if (num_pairs < 0) return PA_ERR_INVALID_ARG;
    if (num_pairs == 0) return PA_OK;
    if (!k_cache || !v_cache || !pairs) return PA_ERR_INVALID_ARG;
    if (!aligned(k_cache, 16) || !aligned(v_cache, 16) || !aligned(pairs, 4))
        return PA_ERR_INVALID_ARG;
    return from_hip(pkv::launch_copy_blocks(d->dtype, d->head_dim, d->block_size, d->num_kv_heads,
                                            d->num_blocks, k_cache, v_cache, pairs, num_pairs,
                                            static_cast<hipStream_t>(stream)));
}

pa_status pa_swap_blocks(const pa_cache_desc* d, const void* src_k, const void* src_v,
                         int32_t src_blocks, void* dst_k, void* dst_v, int32_t dst_blocks,
                         const int32_t* pairs, int32_t num_pairs, void* stream) {
    pa_status st = check_desc(d);
    if (st != PA_OK) return st;
    if (num_pairs < 0 || src_blocks < 0 || dst_blocks < 0) return PA_ERR_INVALID_ARG;
    if (num_pairs == 0) return PA_OK;
    if (!src_k || !src_v || !dst_k || !dst_v || !pairs) return PA_ERR_INVALID_ARG;
    if (!aligned(src_k, 16) || !aligned(src_v, 16) || !aligned(dst_k, 16) || !aligned(dst_v, 16) ||
        !aligned(pairs, 4))
        return PA_ERR_INVALID_ARG;
    if (num_pairs > 2147483647 / 2) return PA_ERR_UNSUPPORTED;
    return from_hip(pkv::launch_swap_blocks(d->dtype, d->head_dim, d->block_size, d->num_kv_heads,
                                            src_k, src_v, src_blocks, dst_k, dst_v, dst_blocks,
                                            pairs, num_pairs, static_cast<hipStream_t>(stream)));
}

pa_status pa_append_tokens(const pa_cache_desc* d, const void* k, const void* v,
                           const int64_t* slot_mapping, const int32_t* cow_pairs,
                           int32_t num_tokens, void* k_cache, void* v_cache,
                           int32_t* block_tables, int32_t num_rows, int32_t max_blocks_per_seq,
                           const int32_t* table_updates, int32_t num_updates,
                           const int32_t* lens_in, int32_t* lens_out, int32_t num_lens,
                           void* stream) {
    pa_status st = check_desc(d);
    if (st != PA_OK) return st;
    if (num_tokens < 0 || num_updates < 0 || num_rows < 0 || max_blocks_per_seq < 0 ||
        num_lens < 0)
        return PA_ERR_INVALID_ARG;
    if (num_tokens == 0 && num_updates == 0 && num_lens == 0) return PA_OK;
    if (num_tokens > 0) {
        if (!k || !v || !slot_mapping || !k_cache || !v_cache) return PA_ERR_INVALID_ARG;
        if (!aligned(k, 16) || !aligned(v, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
            !aligned(slot_mapping, 8) || (cow_pairs && !aligned(cow_pairs, 4)))
            return PA_ERR_INVALID_ARG;
        if (num_tokens > 2147483647 / 4 || d->num_kv_heads > 65535) return PA_ERR_UNSUPPORTED;
    }
    if (num_updates > 0 && (!block_tables || !table_updates || !aligned(block_tables, 4) ||
                            !aligned(table_updates, 4)))
        return PA_ERR_INVALID_ARG;
    if (num_lens > 0 && (!lens_in || !lens_out || !aligned(lens_in, 4) || !aligned(lens_out, 4)))
        return PA_ERR_INVALID_ARG;
    return from_hip(pkv::launch_append_tokens(
        d->dtype, d->head_dim, d->block_size, d->num_kv_heads, d->num_blocks, k, v, slot_mapping,
        num_tokens > 0 ? cow_pairs : nullptr, num_tokens, k_cache, v_cache, block_tables, num_rows,
        max_blocks_per_seq, table_updates, num_updates, lens_in, lens_out, num_lens,
        static_cast<hipStream_t>(stream)));
}

pa_status pa_update_block_tables(int32_t* block_tables, int32_t num_rows,
                                 int32_t max_blocks_per_seq, const int32_t* updates,
                                 int32_t num_updates, void* stream) {
    if (num_rows < 0 || max_blocks_per_seq < 0 || num_updates < 0) return PA_ERR_INVALID_ARG;
    if (num_updates == 0) return PA_OK;
    if (!block_tables || !updates || !aligned(block_tables, 4) || !aligned(updates, 4))
        return PA_ERR_INVALID_ARG;
    return from_hip(pkv::launch_update_block_tables(block_tables, num_rows, max_blocks_per_seq,
                                                    updates, num_updates,
                                                    static_cast<hipStream_t>(stream)));
}

int32_t pa_decode_default_units(void) {
    int32_t u = g_default_units.load();
    if (u > 0) return u;
    int dev = 0, cus = 0;
    if (hipGetDevice(&dev) != hipSuccess ||
        hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0) {
        (void)hipGetLastError();
        cus = 256;
    }
    // Eight one-wave units per CU: with eight KV heads (or query heads) per row
    // group this is one eight-wave workgroup per CU, 16 MiB of K/V reads in flight
    // at one tile per wave; the measured optimum of pass 1 on MI355X (256 CUs ->
    // 2048).
    u = cus * 8;
    g_default_units.store(u);
    return u;
}

size_t pa_decode_workspace_bytes(const pa_cache_desc* d, int32_t num_q_heads, int32_t num_units) {
    if (check_desc(d) != PA_OK || num_q_heads <= 0 || num_q_heads % d->num_kv_heads != 0 ||
        num_units < 0 || num_units > kMaxUnits)
        return 0;
    const int32_t units = num_units == 0 ? pa_decode_default_units() : num_units;
    return workspace_for(d, num_q_heads, units);
}

}  // extern "C"

// ---------------------------------------------------------------------------------
// The static scratch buffer of pa_paged_attn_decode_noalloc: one per GPU the library
// runs on, held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address is looked up once per device
// (with that device current) and only that address is ever passed to kernels.
static __device__ __align__(256) unsigned char scratch[PA_DECODE_NOALLOC_SCRATCH_BYTES];

namespace {

constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices] = {};

__global__ __launch_bounds__(256) void zero_words(uint32_t* __restrict__ p, size_t n) {
    for (size_t i = static_cast<size_t>(blockIdx.x) * 256 + threadIdx.x; i < n;
         i += static_cast<size_t>(gridDim.x) * 256)
        p[i] = 0u;
}

// The current device's copy of `scratch`.  The first call on a device looks up its
// address and zero-fills it with a kernel on `stream` (a fill kernel rather than a
// memset node, so that a caller may capture the call); the arrival counts at its end
// then start at zero, and every completed decode leaves them zero again.
pa_status static_scratch(hipStream_t stream, void** out) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return PA_ERR_HIP;
    }
    if (dev < 0 || dev >= kMaxDevices) return PA_ERR_UNSUPPORTED;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void* p = nullptr;
        const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (e != hipSuccess || !p) {
            (void)hipGetLastError();
            return PA_ERR_HIP;
        }
        const size_t words = PA_DECODE_NOALLOC_SCRATCH_BYTES / 4;
        hipLaunchKernelGGL(zero_words, dim3(1024), dim3(256), 0, stream, static_cast<uint32_t*>(p),
                           words);
        if (hipGetLastError() != hipSuccess) return PA_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *out = g_scratch_ptr[dev];
    return PA_OK;
}

}  // namespace

namespace {

// The step's writes that pa_decode_step folds into the decode launch.
struct StepIO {
    const void* k_new;
    const void* v_new;
    const int64_t* slots;
    const int32_t* cow;
    const int32_t* lens_in;
};

// Validation and argument packing shared by the decode entry points.  With
// use_scratch the workspace arguments are ignored and the library's static
// scratch buffer serves instead (after the request is checked against its size).
// With step, the call is a decode step (pa_decode_step): one launch that also
// performs the step's cache writes.
pa_status decode_call(const pa_cache_desc* d, void* out, const void* q, const void* k_cache,
                      const void* v_cache, const int32_t* block_tables,
                      const int32_t* context_lens, int32_t num_seqs, int32_t num_q_heads,
                      int32_t max_blocks_per_seq, float scale, int32_t num_units, void* workspace,
                      size_t workspace_bytes, uint32_t flags, void* stream, int passes,
                      bool use_scratch = false, const StepIO* step = nullptr) {
    pa_status st = check_desc(d);
    if (st != PA_OK) return st;
    if ((flags & ~static_cast<uint32_t>(PA_DECODE_KEEP_CACHED)) != 0) return PA_ERR_INVALID_ARG;
    if (num_seqs < 0 || num_q_heads <= 0 || max_blocks_per_seq < 0 || num_units < 0 ||
        num_units > kMaxUnits)
        return PA_ERR_INVALID_ARG;
    if (num_q_heads % d->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
    const int32_t group = num_q_heads / d->num_kv_heads;
    const bool use_group = group_kernel_for(d, group);
    if (use_group && group != 2 && group != 4 && group != 8 && group != 16)
        return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0) return PA_OK;
    if (max_blocks_per_seq == 0) return PA_ERR_INVALID_ARG;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !context_lens ||
        (!use_scratch && !workspace))
        return PA_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        (!use_scratch && !aligned(workspace, 16)) || !aligned(block_tables, 4) ||
        !aligned(context_lens, 4))
        return PA_ERR_INVALID_ARG;
    if (step) {
        if (!step->k_new || !step->v_new || !step->slots || !step->lens_in ||
            !aligned(step->k_new, 16) || !aligned(step->v_new, 16) || !aligned(step->slots, 8) ||
            !aligned(step->lens_in, 4) || (step->cow && !aligned(step->cow, 4)))
            return PA_ERR_INVALID_ARG;
    }
    const int32_t units = num_units == 0 ? pa_decode_default_units() : num_units;
    const size_t need = workspace_layout(d, num_q_heads, units, step ? num_seqs : -1).bytes;
    if (use_scratch) {
        if (need > PA_DECODE_NOALLOC_SCRATCH_BYTES) return PA_ERR_TOO_LARGE;
    } else if (workspace_bytes < need) {
        return PA_ERR_INVALID_ARG;
    }
    // tiles of the cache layout per block (a block of 8 tokens is one 8-token tile)
    const int32_t tpb = d->block_size >= pkv::kTile ? d->block_size / pkv::kTile : 1;
    const int32_t rows = use_group ? d->num_kv_heads : num_q_heads;
    // Every tile position of the batch (rows x sequences x table columns) must fit in int32.
    const double positions = static_cast<double>(rows) * num_seqs * max_blocks_per_seq * tpb;
    if (positions + units >= 2147483647.0) return PA_ERR_UNSUPPORTED;
    // Tile indices into the cache (block * Hkv + head) * tpb + tile are int32 in the kernels.
    if (static_cast<double>(d->num_blocks) * d->num_kv_heads * tpb >= 2147483647.0)
        return PA_ERR_UNSUPPORTED;

    if (use_scratch) {
        const pa_status ss = static_scratch(static_cast<hipStream_t>(stream), &workspace);
        if (ss != PA_OK) return ss;
        workspace_bytes = PA_DECODE_NOALLOC_SCRATCH_BYTES;
    }

    pkv::DecodeArgs a;
    a.q = q;
    a.out = out;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.context_lens = context_lens;
    {
        const WorkspaceLayout w = workspace_layout(d, num_q_heads, units, step ? num_seqs : -1);
        char* base = static_cast<char*>(workspace);
        a.pieces = reinterpret_cast<float*>(base);
        a.unit_rec = reinterpret_cast<int32_t*>(base + w.rec_offset);
        a.split_count_end = reinterpret_cast<int32_t*>(base + (workspace_bytes & ~size_t(3)));
        a.heads_per_row = use_group ? group : 1;
        a.lens_in = step ? step->lens_in : nullptr;
        a.new_slots = step ? step->slots : nullptr;
        a.cow_in = step ? step->cow : nullptr;
        a.k_new = step ? step->k_new : nullptr;
        a.v_new = step ? step->v_new : nullptr;
        a.lens_dev = step ? const_cast<int32_t*>(context_lens) : nullptr;
        a.tables_dev = step ? const_cast<int32_t*>(block_tables) : nullptr;
        a.sync = step ? reinterpret_cast<int32_t*>(base + w.step_offset) : nullptr;
        a.seq_info = step ? reinterpret_cast<int32_t*>(base + w.step_offset + 16) : nullptr;
        a.block_size = d->block_size;
    }
    a.num_seqs = num_seqs;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = d->num_kv_heads;
    a.group = group;
    a.rows = rows;
    a.max_blocks = max_blocks_per_seq;
    a.tiles_per_block = tpb;
    a.num_blocks = d->num_blocks;
    // Aligned split: with at least one unit per row, every row is cut into the same
    // ranges, and the rows of a range (up to 8, a power of two dividing the row
    // count) share a workgroup.
    a.fused = (passes == 3 || step) ? 1 : 0;
    a.keep_cached = (flags & PA_DECODE_KEEP_CACHED) ? 1 : 0;

    a.num_units = units;
    a.aligned = units >= rows ? 1 : 0;
    a.waves_per_group = 1;
    if (a.aligned)
        while (a.waves_per_group < 8 && rows % (2 * a.waves_per_group) == 0) a.waves_per_group *= 2;
    a.scale_log2e = scale * 1.4426950408889634f;
    if (step)
        return from_hip(pkv::launch_decode_step(d->dtype, d->head_dim, use_group, a,
                                                static_cast<hipStream_t>(stream)));
    return from_hip(pkv::launch_decode(d->dtype, d->head_dim, use_group, a, passes,
                                       static_cast<hipStream_t>(stream)));
}

}  // namespace

extern "C" {

pa_status pa_paged_attn_decode(const pa_cache_desc* d, void* out, const void* q,
                               const void* k_cache, const void* v_cache,
                               const int32_t* block_tables, const int32_t* context_lens,
                               int32_t num_seqs, int32_t num_q_heads,
                               int32_t max_blocks_per_seq, float scale, int32_t num_units,
                               void* workspace, size_t workspace_bytes, uint32_t flags,
                               void* stream) {
    return decode_call(d, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                       num_q_heads, max_blocks_per_seq, scale, num_units, workspace,
                       workspace_bytes, flags, stream, 3);
}

pa_status pa_paged_attn_decode_partial(const pa_cache_desc* d, void* out, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       int32_t max_blocks_per_seq, float scale,
                                       int32_t num_units, void* workspace,
                                       size_t workspace_bytes, uint32_t flags, void* stream) {
    return decode_call(d, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                       num_q_heads, max_blocks_per_seq, scale, num_units, workspace,
                       workspace_bytes, flags, stream, 1);
}

size_t pa_decode_step_workspace_bytes(const pa_cache_desc* d, int32_t num_q_heads,
                                      int32_t num_units, int32_t num_seqs) {
    if (check_desc(d) != PA_OK || num_q_heads <= 0 || num_q_heads % d->num_kv_heads != 0 ||
        num_units < 0 || num_units > kMaxUnits || num_seqs < 0)
        return 0;
    const int32_t units = num_units == 0 ? pa_decode_default_units() : num_units;
    return workspace_layout(d, num_q_heads, units, num_seqs).bytes;
}

pa_status pa_decode_step(const pa_cache_desc* d, void* out, const void* q, const void* k_new,
                         const void* v_new, const int64_t* slot_mapping, const int32_t* cow_pairs,
                         const int32_t* lens_in, void* k_cache, void* v_cache,
                         int32_t* block_tables, int32_t* context_lens, int32_t num_seqs,
                         int32_t num_q_heads, int32_t max_blocks_per_seq, float scale,
                         int32_t num_units, void* workspace, size_t workspace_bytes,
                         uint32_t flags, void* stream) {
    const StepIO io{k_new, v_new, slot_mapping, cow_pairs, lens_in};
    return decode_call(d, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                       num_q_heads, max_blocks_per_seq, scale, num_units, workspace,
                       workspace_bytes, flags, stream, 3, false, &io);
}

pa_status pa_paged_attn_decode_noalloc(const pa_cache_desc* d, void* out, const void* q,
                                       const void* k_cache, const void* v_cache,
                                       const int32_t* block_tables, const int32_t* context_lens,
                                       int32_t num_seqs, int32_t num_q_heads,
                                       int32_t max_blocks_per_seq, float scale,
                                       int32_t num_units, uint32_t flags, void* stream) {
    return decode_call(d, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                       num_q_heads, max_blocks_per_seq, scale, num_units, nullptr, 0, flags,
                       stream, 3, /*use_scratch=*/true);
}

pa_status pa_paged_attn_decode_merge(const pa_cache_desc* d, void* out, const void* q,
                                     const void* k_cache, const void* v_cache,
                                     const int32_t* block_tables, const int32_t* context_lens,
                                     int32_t num_seqs, int32_t num_q_heads,
                                     int32_t max_blocks_per_seq, float scale, int32_t num_units,
                                     void* workspace, size_t workspace_bytes, uint32_t flags,
                                     void* stream) {
    return decode_call(d, out, q, k_cache, v_cache, block_tables, context_lens, num_seqs,
                       num_q_heads, max_blocks_per_seq, scale, num_units, workspace,
                       workspace_bytes, flags, stream, 2);
}

pa_status pa_paged_attn_prefill(const pa_cache_desc* d, void* out, const void* q,
                                const void* k_cache, const void* v_cache,
                                const int32_t* block_tables, const int32_t* query_start,
                                const int32_t* context_lens, int32_t num_seqs,
                                int32_t num_tokens, int32_t num_q_heads,
                                int32_t max_blocks_per_seq, int32_t max_query_len, float scale,
                                void* stream) {
    pa_status st = check_desc(d);
    if (st != PA_OK) return st;
    if (num_seqs < 0 || num_tokens < 0 || num_q_heads <= 0 || max_blocks_per_seq < 0 ||
        max_query_len < 0)
        return PA_ERR_INVALID_ARG;
    if (num_q_heads % d->num_kv_heads != 0) return PA_ERR_INVALID_ARG;
    if (!std::isfinite(scale)) return PA_ERR_INVALID_ARG;
    const int32_t group = num_q_heads / d->num_kv_heads;
    if (d->dtype != PA_DTYPE_BF16 || 16 % group != 0) return PA_ERR_UNSUPPORTED;
    if (num_seqs == 0 || num_tokens == 0 || max_query_len == 0) return PA_OK;
    if (max_blocks_per_seq == 0) return PA_ERR_INVALID_ARG;
    if (!out || !q || !k_cache || !v_cache || !block_tables || !query_start || !context_lens)
        return PA_ERR_INVALID_ARG;
    if (!aligned(out, 16) || !aligned(q, 16) || !aligned(k_cache, 16) || !aligned(v_cache, 16) ||
        !aligned(block_tables, 4) || !aligned(query_start, 4) || !aligned(context_lens, 4))
        return PA_ERR_INVALID_ARG;
    const int32_t tpb = d->block_size >= pkv::kTile ? d->block_size / pkv::kTile : 1;
    // int32 in the kernel: cache tile indices, positions, and the workgroup count
    // (at most (num_seqs * Hkv + 7) * (max_query_len / 8 + 1))
    if (static_cast<double>(d->num_blocks) * d->num_kv_heads * tpb >= 2147483647.0 ||
        static_cast<double>(max_blocks_per_seq) * d->block_size >= 2147483647.0 ||
        (static_cast<double>(num_seqs) * d->num_kv_heads + 8) * (max_query_len / 8.0 + 2) >=
            2147483647.0)
        return PA_ERR_UNSUPPORTED;
    pkv::PrefillArgs a;
    a.q = q;
    a.out = out;
    a.k_cache = k_cache;
    a.v_cache = v_cache;
    a.block_tables = block_tables;
    a.query_start = query_start;
    a.context_lens = context_lens;
    a.num_seqs = num_seqs;
    a.num_tokens = num_tokens;
    a.num_q_heads = num_q_heads;
    a.num_kv_heads = d->num_kv_heads;
    a.max_blocks = max_blocks_per_seq;
    a.tiles_per_block = tpb;
    a.num_blocks = d->num_blocks;
    a.qgroups = 0;
    a.num_groups = 0;
    a.block_size = d->block_size;
    a.scale_log2e = scale * 1.4426950408889634f;
    return from_hip(pkv::launch_prefill(d->head_dim, group, max_query_len, a,
                                        static_cast<hipStream_t>(stream)));
}

}  // extern "C"
