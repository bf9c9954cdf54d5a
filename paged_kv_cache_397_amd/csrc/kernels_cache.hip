// Cache-side kernels: scatter of new tokens into their slots, whole-block copy,
// and in-place block-table updates.  All three are pure data movement (bits in,
// bits out); the physical layout they write is the one declared in pagedkv.h.

#include "pagedkv_internal.h"

namespace pkv {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

// One workgroup per (token, kv head); one thread per head-dim position.
// Writing new tokens into the slots of their blocks is the "scatter" half of
// paged KV access (ksqn.cn "大模型推理性能优化：PagedAttention与Continuous
// Batching原理与实践", section 2.2).  Thread d stores V element d; threads with
// d % X == 0 also copy the 16-byte K group of dims d .. d+X-1.
template <typename T, int D>
__global__ __launch_bounds__(D) void reshape_and_cache_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const int64_t* __restrict__ slots,
    T* __restrict__ k_cache, T* __restrict__ v_cache, int num_kv_heads, int block_size,
    int64_t num_slots) {
    constexpr int X = 16 / sizeof(T);  // elements per 16-byte group
    constexpr int E = X / 4;           // dims per 16-byte V group
    const int t = blockIdx.x;
    const int h = blockIdx.y;
    const int d = threadIdx.x;
    const int64_t slot = slots[t];
    if (slot < 0 || slot >= num_slots) return;
    const int64_t b = slot / block_size;
    const int o = static_cast<int>(slot - b * block_size);
    const int tpb = block_size / kTile;
    const size_t tile_base =
        ((static_cast<size_t>(b) * tpb + (o >> 4)) * num_kv_heads + h) * (kTile * D);
    const size_t src = (static_cast<size_t>(t) * num_kv_heads + h) * D;
    const int ti = o & 15;
    // V: 16-byte group (m, j, i) holds tokens 4j..4j+3 of dims 16E*m + 16e + i.
    const int m = d / (16 * E);
    const int e = (d >> 4) % E;
    const int i = d & 15;
    const int j = ti >> 2;
    const int r = ti & 3;
    v_cache[tile_base + ((((m * 4 + j) * 16 + i) * E + e) * 4 + r)] = v[src + d];
    // K: 16-byte group (c, token) holds dims c*X .. c*X+X-1 of one token.
    if (d % X == 0) {
        const int c = d / X;
        *reinterpret_cast<u32x4*>(k_cache + tile_base + (c * 16 + ti) * X) =
            *reinterpret_cast<const u32x4*>(k + src + d);
    }
}

// Grid (pairs, 2 arrays, chunks); 256 threads copy 16 bytes each per chunk.
__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4* __restrict__ k_cache,
                                                          u32x4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_blocks, int64_t block_u4) {
    const int src = pairs[2 * blockIdx.x];
    const int dst = pairs[2 * blockIdx.x + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    u32x4* base = blockIdx.y == 0 ? k_cache : v_cache;
    const int64_t n = static_cast<int64_t>(blockIdx.z) * 1024 + threadIdx.x;
    const u32x4* s = base + src * block_u4;
    u32x4* dp = base + dst * block_u4;
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t idx = n + k * 256;
        if (idx < block_u4) dp[idx] = s[idx];
    }
}

// Whole-block copies between two pools of the same block geometry - HBM and pinned
// host memory for swapping a suspended sequence out and back (hihuo.com "vLLM 原理：
// PagedAttention 和 Continuous Batching", Preemption（抢占）: the Swap mode).  A block
// is one contiguous region of each cache array; workgroup (pair, K or V, chunk)
// moves 16 KiB with four 16-B loads in flight per thread, so that many requests
// cross the host link at once.  Pairs naming a block outside its pool are skipped.
__global__ __launch_bounds__(256) void swap_blocks_kernel(const u32x4* __restrict__ src_k,
                                                          const u32x4* __restrict__ src_v,
                                                          u32x4* __restrict__ dst_k,
                                                          u32x4* __restrict__ dst_v,
                                                          const int32_t* __restrict__ pairs,
                                                          int src_blocks, int dst_blocks,
                                                          int64_t block_u4) {
    const int src = pairs[2 * blockIdx.x];
    const int dst = pairs[2 * blockIdx.x + 1];
    if (src < 0 || src >= src_blocks || dst < 0 || dst >= dst_blocks) return;
    const u32x4* s = (blockIdx.y == 0 ? src_k : src_v) + src * block_u4;
    u32x4* d = (blockIdx.y == 0 ? dst_k : dst_v) + dst * block_u4;
    const int64_t n = static_cast<int64_t>(blockIdx.z) * 1024 + threadIdx.x;
    u32x4 r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t idx = n + k * 256;
        if (idx < block_u4) r[k] = s[idx];
    }
#pragma unroll
    for (int k = 0; k < 4; ++k) {
        const int64_t idx = n + k * 256;
        if (idx < block_u4) d[idx] = r[k];
    }
}

__global__ __launch_bounds__(256) void update_tables_kernel(int32_t* __restrict__ tables, int rows,
                                                            int cols,
                                                            const int32_t* __restrict__ upd,
                                                            int n) {
    const int k = blockIdx.x * 256 + threadIdx.x;
    if (k >= n) return;
    const int r = upd[3 * k];
    const int c = upd[3 * k + 1];
    if (r < 0 || r >= rows || c < 0 || c >= cols) return;
    tables[static_cast<int64_t>(r) * cols + c] = upd[3 * k + 2];
}

// One decode step's writes in one launch.  Workgroup (t, h) first copies KV head
// h's part of the block that token t's copy-on-write pair names (if any), then
// scatters token t's K and V for head h; every workgroup applies its share of the
// block-table updates and of the context-length copy.  A head's part of a block is
// its tile in each of the block's tile slots (tiles are ordered block -> tile ->
// head), so the copy and the token's write for that head never leave the workgroup.
// Another token's in-place write into the copy source can land before the copy
// reads it; it is then carried into the copy at the offset the copying token itself
// writes next (sequences that share a block hold the same number of tokens in it),
// so the final bytes equal copy-all, then write-all.  The metadata arrays may live
// in pinned host memory: each element is read once.
template <typename T, int D>
__global__ __launch_bounds__(D) void append_tokens_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const int64_t* __restrict__ slots,
    const int32_t* __restrict__ cow, int num_tokens, T* __restrict__ k_cache,
    T* __restrict__ v_cache, int num_kv_heads, int block_size, int num_blocks,
    int32_t* __restrict__ tables, int rows, int cols, const int32_t* __restrict__ upd,
    int num_updates, const int32_t* __restrict__ lens_in, int32_t* __restrict__ lens_out,
    int num_lens) {
    constexpr int X = 16 / sizeof(T);
    constexpr int E = X / 4;
    const int t = blockIdx.x, h = blockIdx.y;
    const int tid = threadIdx.x;
    const int wg = blockIdx.y * gridDim.x + blockIdx.x;
    const int nwg = gridDim.x * gridDim.y;
    // Every metadata element this thread needs is requested before any is used: read
    // from pinned host memory, each dependent read would cost a host-link round trip.
    const bool tok = t < num_tokens;
    const int64_t slot = tok ? slots[t] : -1;
    const int cow_src = (tok && cow) ? cow[2 * t] : -1;
    const int cow_dst = (tok && cow) ? cow[2 * t + 1] : -1;
    const int n0 = wg * D + tid;
    const int ur = n0 < num_updates ? upd[3 * n0] : -1;
    const int uc = n0 < num_updates ? upd[3 * n0 + 1] : -1;
    const int ub = n0 < num_updates ? upd[3 * n0 + 2] : 0;
    const int ln = n0 < num_lens ? lens_in[n0] : 0;
    if (ur >= 0 && ur < rows && uc >= 0 && uc < cols) tables[static_cast<int64_t>(ur) * cols + uc] = ub;
    if (n0 < num_lens) lens_out[n0] = ln;
    for (int n = n0 + nwg * D; n < num_updates; n += nwg * D) {  // more entries than threads
        const int r = upd[3 * n], c = upd[3 * n + 1];
        if (r >= 0 && r < rows && c >= 0 && c < cols) tables[static_cast<int64_t>(r) * cols + c] = upd[3 * n + 2];
    }
    for (int n = n0 + nwg * D; n < num_lens; n += nwg * D) lens_out[n] = lens_in[n];
    if (!tok) return;
    const int tpb = block_size / kTile;
    constexpr int tile_u4 = kTile * D * static_cast<int>(sizeof(T)) / 16;  // one tile of one head
    if (cow) {
        if (cow_src >= 0 && cow_src < num_blocks && cow_dst >= 0 && cow_dst < num_blocks &&
            cow_src != cow_dst) {
            // head h's part of a block: its tile in each of the block's tpb tile slots
            for (int tt = 0; tt < tpb; ++tt) {
                const int64_t so = ((static_cast<int64_t>(cow_src) * tpb + tt) * num_kv_heads + h) * tile_u4;
                const int64_t dof = ((static_cast<int64_t>(cow_dst) * tpb + tt) * num_kv_heads + h) * tile_u4;
                const u32x4* ks = reinterpret_cast<const u32x4*>(k_cache) + so;
                const u32x4* vs = reinterpret_cast<const u32x4*>(v_cache) + so;
                u32x4* kd = reinterpret_cast<u32x4*>(k_cache) + dof;
                u32x4* vd = reinterpret_cast<u32x4*>(v_cache) + dof;
                for (int i = tid; i < tile_u4; i += D) {
                    kd[i] = ks[i];
                    vd[i] = vs[i];
                }
            }
            // the copy's stores complete before any thread writes the token over them
            __builtin_amdgcn_s_waitcnt(0x0F70);
        }
        __syncthreads();
    }
    if (slot < 0 || slot >= static_cast<int64_t>(num_blocks) * block_size) return;
    const int64_t b = slot / block_size;
    const int o = static_cast<int>(slot - b * block_size);
    const int ti = o & 15;
    const int j = ti >> 2, r = ti & 3;
    const int d = tid;
    const size_t tile_base =
        ((static_cast<size_t>(b) * tpb + (o >> 4)) * num_kv_heads + h) * (kTile * D);
    const size_t src = (static_cast<size_t>(t) * num_kv_heads + h) * D;
    const int m = d / (16 * E), ee = (d >> 4) % E, i = d & 15;
    v_cache[tile_base + ((((m * 4 + j) * 16 + i) * E + ee) * 4 + r)] = v[src + d];
    if (d % X == 0)
        *reinterpret_cast<u32x4*>(k_cache + tile_base + ((d / X) * 16 + ti) * X) =
            *reinterpret_cast<const u32x4*>(k + src + d);
}

template <typename T, int D>
hipError_t launch_append(const void* k, const void* v, const int64_t* slots, const int32_t* cow,
                         int num_tokens, void* kc, void* vc, int hkv, int bs, int nb,
                         int32_t* tables, int rows, int cols, const int32_t* upd, int n_upd,
                         const int32_t* lens_in, int32_t* lens_out, int n_lens, hipStream_t st) {
    const int extra = (n_upd > n_lens ? n_upd : n_lens);
    const dim3 grid = num_tokens > 0 ? dim3(num_tokens, hkv) : dim3((extra + D - 1) / D, 1);
    if (grid.x == 0) return hipSuccess;
    hipLaunchKernelGGL((append_tokens_kernel<T, D>), grid, dim3(D), 0, st,
                       static_cast<const T*>(k), static_cast<const T*>(v), slots, cow, num_tokens,
                       static_cast<T*>(kc), static_cast<T*>(vc), hkv, bs, nb, tables, rows, cols,
                       upd, n_upd, lens_in, lens_out, n_lens);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_rc(const void* k, const void* v, const int64_t* slots, int num_tokens,
                     void* kc, void* vc, int hkv, int bs, int nb, hipStream_t st) {
    dim3 grid(num_tokens, hkv);
    hipLaunchKernelGGL((reshape_and_cache_kernel<T, D>), grid, dim3(D), 0, st,
                       static_cast<const T*>(k), static_cast<const T*>(v), slots,
                       static_cast<T*>(kc), static_cast<T*>(vc), hkv, bs,
                       static_cast<int64_t>(nb) * bs);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_reshape_and_cache(int dtype, int head_dim, int block_size, int num_kv_heads,
                                    int num_blocks, const void* k, const void* v,
                                    const int64_t* slots, int num_tokens, void* k_cache,
                                    void* v_cache, hipStream_t stream) {
    const bool f32 = dtype == 0;
    if (head_dim == 64)
        return f32 ? launch_rc<uint32_t, 64>(k, v, slots, num_tokens, k_cache, v_cache,
                                             num_kv_heads, block_size, num_blocks, stream)
                   : launch_rc<uint16_t, 64>(k, v, slots, num_tokens, k_cache, v_cache,
                                             num_kv_heads, block_size, num_blocks, stream);
    if (head_dim == 128)
        return f32 ? launch_rc<uint32_t, 128>(k, v, slots, num_tokens, k_cache, v_cache,
                                              num_kv_heads, block_size, num_blocks, stream)
                   : launch_rc<uint16_t, 128>(k, v, slots, num_tokens, k_cache, v_cache,
                                              num_kv_heads, block_size, num_blocks, stream);
    return hipErrorInvalidValue;
}

hipError_t launch_append_tokens(int dtype, int head_dim, int block_size, int num_kv_heads,
                                int num_blocks, const void* k, const void* v,
                                const int64_t* slots, const int32_t* cow, int num_tokens,
                                void* k_cache, void* v_cache, int32_t* tables, int rows, int cols,
                                const int32_t* upd, int num_updates, const int32_t* lens_in,
                                int32_t* lens_out, int num_lens, hipStream_t stream) {
    const bool f32 = dtype == 0;
#define PKV_APPEND(T, D)                                                                      \
    launch_append<T, D>(k, v, slots, cow, num_tokens, k_cache, v_cache, num_kv_heads,       \
                        block_size, num_blocks, tables, rows, cols, upd, num_updates,        \
                        lens_in, lens_out, num_lens, stream)
    if (head_dim == 64) return f32 ? PKV_APPEND(uint32_t, 64) : PKV_APPEND(uint16_t, 64);
    if (head_dim == 128) return f32 ? PKV_APPEND(uint32_t, 128) : PKV_APPEND(uint16_t, 128);
#undef PKV_APPEND
    return hipErrorInvalidValue;
}

hipError_t launch_copy_blocks(int dtype, int head_dim, int block_size, int num_kv_heads,
                              int num_blocks, void* k_cache, void* v_cache, const int32_t* pairs,
                              int num_pairs, hipStream_t stream) {
    const int64_t elem = dtype == 0 ? 4 : 2;
    const int64_t block_u4 = static_cast<int64_t>(num_kv_heads) * block_size * head_dim * elem / 16;
    const int64_t chunks = (block_u4 + 1023) / 1024;
    dim3 grid(num_pairs, 2, static_cast<unsigned>(chunks));
    hipLaunchKernelGGL(copy_blocks_kernel, grid, dim3(256), 0, stream,
                       static_cast<u32x4*>(k_cache), static_cast<u32x4*>(v_cache), pairs,
                       num_blocks, block_u4);
    return hipGetLastError();
}

hipError_t launch_swap_blocks(int dtype, int head_dim, int block_size, int num_kv_heads,
                              const void* src_k, const void* src_v, int src_blocks, void* dst_k,
                              void* dst_v, int dst_blocks, const int32_t* pairs, int num_pairs,
                              hipStream_t stream) {
    const int64_t block_u4 = static_cast<int64_t>(num_kv_heads) * block_size * head_dim *
                             (dtype == 0 ? 4 : 2) / 16;
    const dim3 grid(num_pairs, 2, static_cast<unsigned>((block_u4 + 1023) / 1024));
    hipLaunchKernelGGL(swap_blocks_kernel, grid, dim3(256), 0, stream,
                       static_cast<const u32x4*>(src_k), static_cast<const u32x4*>(src_v),
                       static_cast<u32x4*>(dst_k), static_cast<u32x4*>(dst_v), pairs, src_blocks,
                       dst_blocks, block_u4);
    return hipGetLastError();
}

hipError_t launch_update_block_tables(int32_t* tables, int rows, int cols, const int32_t* upd,
                                      int n, hipStream_t stream) {
    hipLaunchKernelGGL(update_tables_kernel, dim3((n + 255) / 256), dim3(256), 0, stream, tables,
                       rows, cols, upd, n);
    return hipGetLastError();
}

}  // namespace pkv
