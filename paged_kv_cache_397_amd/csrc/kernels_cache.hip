// Cache-side kernels: scatter of new tokens into their slots, whole-block copy,
// and in-place block-table updates.  All three are pure data movement (bits in,
// bits out); the physical layout they write is the one declared in pagedkv.h.

#include "pagedkv_internal.h"

namespace pkv {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
constexpr int kWaveSize = 64;

// Lane `lane`'s 64-bit value; the low half is taken unsigned, so offsets of 2^31
// elements and more (caches over 4 GiB of bf16) keep their value.
__device__ __forceinline__ long long readlane_i64(long long x, int lane) {
    const unsigned lo = static_cast<unsigned>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<unsigned long long>(x)), lane));
    const unsigned hi = static_cast<unsigned>(
        __builtin_amdgcn_readlane(static_cast<int>(static_cast<unsigned long long>(x) >> 32), lane));
    return static_cast<long long>((static_cast<unsigned long long>(hi) << 32) | lo);
}

// Writing new tokens into the slots of their blocks is the "scatter" half of paged
// KV access (ksqn.cn "大模型推理性能优化：PagedAttention与Continuous Batching原理与实践",
// section 2.2).  One wavefront per (window of 16 consecutive tokens, kv head).
//
// A V 16-byte group holds four consecutive slots (4j .. 4j+3 of a tile) of E dims,
// so a single token can only write 2- or 4-byte pieces of it.  Tokens k .. k+3 of
// the window whose slots are s .. s+3 with s a multiple of 4 (a prompt chunk's
// tokens get consecutive slots, wherever the chunk starts in the batch) fill whole
// groups: the window's V rows are staged in LDS and each such quad's groups are
// stored as 16-byte writes.  Tokens in no such quad are written element by
// element.  K groups hold one token each and are always 16-byte writes.
template <typename T, int D>
__global__ __launch_bounds__(64) void reshape_and_cache_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const int64_t* __restrict__ slots,
    int num_tokens, T* __restrict__ k_cache, T* __restrict__ v_cache, int num_kv_heads,
    int block_size, int64_t num_slots) {
    constexpr int X = 16 / sizeof(T);  // elements per 16-byte group
    constexpr int E = X / 4;           // dims per 16-byte V group
    constexpr int KG = D / X;          // 16-byte K groups per token (also per V row)
    constexpr int TW = 16;             // tokens per window
    __shared__ __attribute__((aligned(16))) T vrow[TW][D];
    const int t0 = TW * static_cast<int>(blockIdx.x);
    const int h = blockIdx.y;
    const int lane = threadIdx.x;
    const int tt = block_size < kTile ? block_size : kTile;  // tokens per tile (8 or 16)
    const int tshift = __builtin_ctz(static_cast<unsigned>(tt));
    const int tpb = block_size / tt;
    const int bshift = __builtin_ctz(static_cast<unsigned>(block_size));  // a power of two
    // lane k < 16: token t0 + k's slot (-1 = skip), its tile's element offset and slot in tile
    long long my = -1;
    if (lane < TW && t0 + lane < num_tokens) {
        const int64_t sv = slots[t0 + lane];
        my = (sv >= 0 && sv < num_slots) ? sv : -1;
    }
    long long tb = 0;
    int ti = 0;
    if (my >= 0) {
        const long long b = my >> bshift;
        const int o = static_cast<int>(my & (block_size - 1));
        tb = ((b * tpb + (o >> tshift)) * num_kv_heads + h) * static_cast<long long>(tt * D);
        ti = o & (tt - 1);
    }
    const long long n1 = __shfl_down(my, 1), n2 = __shfl_down(my, 2), n3 = __shfl_down(my, 3);
    const bool qstart = lane < TW - 3 && my >= 0 && (my & 3) == 0 && n1 == my + 1 &&
                        n2 == my + 2 && n3 == my + 3;
    const uint32_t qmask = static_cast<uint32_t>(__ballot(qstart));
    const uint32_t valid = static_cast<uint32_t>(__ballot(my >= 0)) & 0xffffu;
    const uint32_t covered = (qmask | (qmask << 1) | (qmask << 2) | (qmask << 3)) & 0xffffu;
    // K of every token, and V rows into LDS: piece `it` of a lane is (token r, 16-byte
    // chunk c).  Every load is issued, unconditionally, before the first store, so a
    // wave has all of its window's reads in flight at once (a loop that stores each
    // piece before loading the next keeps one pair in flight); a row past the last
    // token reads the last token's row instead (in bounds, never stored).
    constexpr int NI = TW * KG / kWaveSize;
    static_assert(NI * kWaveSize == TW * KG, "pieces per lane");
    u32x4 kr[NI], vr[NI];
#pragma unroll
    for (int it = 0; it < NI; ++it) {
        const int g = lane + it * kWaveSize, r = g / KG, c = g % KG;
        const int row = min(t0 + r, num_tokens - 1);
        const size_t src = (static_cast<size_t>(row) * num_kv_heads + h) * D + c * X;
        kr[it] = *reinterpret_cast<const u32x4*>(k + src);
        vr[it] = *reinterpret_cast<const u32x4*>(v + src);
    }
#pragma unroll
    for (int it = 0; it < NI; ++it) {
        const int g = lane + it * kWaveSize, r = g / KG, c = g % KG;
        const long long tbr = __shfl(tb, r);
        const int tir = __shfl(ti, r);
        if ((valid >> r) & 1u) {
            *reinterpret_cast<u32x4*>(k_cache + tbr + (c * tt + tir) * X) = kr[it];
            *reinterpret_cast<u32x4*>(&vrow[r][c * X]) = vr[it];
        }
    }
    __syncthreads();
    // V of each quad: group (m, j, i) holds dims 16E*m + 16e + i (e < E) of its 4 tokens
    const int tq = tt >> 2;  // quads per tile
    for (uint32_t qm = qmask; qm != 0; qm &= qm - 1) {
        const int q = __builtin_ctz(qm);
        const long long tbq = readlane_i64(tb, q);
        const int j = __builtin_amdgcn_readlane(ti, q) >> 2;
        for (int g = lane; g < D / E; g += kWaveSize) {
            const int m = g / 16, i = g % 16;
            u32x4 w;
            if constexpr (sizeof(T) == 2) {
#pragma unroll
                for (int e = 0; e < E; ++e)
#pragma unroll
                    for (int h2 = 0; h2 < 2; ++h2) {
                        const int d = 16 * E * m + 16 * e + i;
                        w[2 * e + h2] = static_cast<uint32_t>(vrow[q + 2 * h2][d]) |
                                        (static_cast<uint32_t>(vrow[q + 2 * h2 + 1][d]) << 16);
                    }
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r) w[r] = static_cast<uint32_t>(vrow[q + r][16 * m + i]);
            }
            *reinterpret_cast<u32x4*>(v_cache + tbq + (((m * tq + j) * 16 + i) * E) * 4) = w;
        }
    }
    // V of the tokens in no quad, element by element
    for (uint32_t um = valid & ~covered; um != 0; um &= um - 1) {
        const int r = __builtin_ctz(um);
        const long long tbr = readlane_i64(tb, r);
        const int tir = __builtin_amdgcn_readlane(ti, r);
        const int j = tir >> 2, rr = tir & 3;
        for (int d = lane; d < D; d += kWaveSize) {
            const int m = d / (16 * E), e = (d >> 4) % E, i = d & 15;
            v_cache[tbr + ((((m * tq + j) * 16 + i) * E + e) * 4 + rr)] = vrow[r][d];
        }
    }
}

// The 16-byte pieces idx = n + 256 k (k < 4) of one block that a thread moves:
// all four loads are issued before the first store (a piece past the block's end
// loads the block's last piece instead, in bounds, and is not stored), so that a
// thread keeps four requests in flight rather than one.
__device__ __forceinline__ void move_four(const u32x4* __restrict__ s, u32x4* __restrict__ d,
                                          int64_t n, int64_t block_u4) {
    u32x4 r[4];
#pragma unroll
    for (int k = 0; k < 4; ++k) r[k] = s[min(n + k * 256, block_u4 - 1)];
    // all four values are taken here, so the compiler cannot sink a load into the
    // store that uses it (it would wait for each in turn)
    asm volatile("" : "+v"(r[0]), "+v"(r[1]), "+v"(r[2]), "+v"(r[3]));
#pragma unroll
    for (int k = 0; k < 4; ++k)
        if (n + k * 256 < block_u4) d[n + k * 256] = r[k];
}

// Grid (pairs, 2 arrays, 16 KiB chunks of a block); each of 256 threads moves four
// 16-byte pieces of its chunk.
__global__ __launch_bounds__(256) void copy_blocks_kernel(u32x4* __restrict__ k_cache,
                                                          u32x4* __restrict__ v_cache,
                                                          const int32_t* __restrict__ pairs,
                                                          int num_blocks, int64_t block_u4) {
    const int src = pairs[2 * blockIdx.x];
    const int dst = pairs[2 * blockIdx.x + 1];
    if (src < 0 || src >= num_blocks || dst < 0 || dst >= num_blocks) return;
    u32x4* base = blockIdx.y == 0 ? k_cache : v_cache;
    const int64_t n = static_cast<int64_t>(blockIdx.z) * 1024 + threadIdx.x;
    if (n >= block_u4) return;
    move_four(base + src * block_u4, base + dst * block_u4, n, block_u4);
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
    const int64_t n = static_cast<int64_t>(blockIdx.z) * 1024 + threadIdx.x;
    if (n >= block_u4) return;
    move_four((blockIdx.y == 0 ? src_k : src_v) + src * block_u4,
              (blockIdx.y == 0 ? dst_k : dst_v) + dst * block_u4, n, block_u4);
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

// One decode step's writes: workgroup (t, h) scatters token t's K and V for head
// h; every workgroup applies its share of the block-table updates and of the
// context-length copy.  Copy-on-write copies, when a step has any, run as a
// launch of their own before this one (launch_append), so every copy reads its
// source before any token of the step is written and no token write can be
// overwritten by a copy: the bytes equal copy-all, then write-all, for any slots
// (several tokens of one sequence in one call included).  The metadata arrays may
// live in pinned host memory: each element is read once.
template <typename T, int D>
__global__ __launch_bounds__(D) void append_tokens_kernel(
    const T* __restrict__ k, const T* __restrict__ v, const int64_t* __restrict__ slots,
    int num_tokens, T* __restrict__ k_cache,
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
    // The token's K and V (device memory) are requested beside the slot (possibly a
    // host-link read), not after it: they do not depend on it.
    const int d = tid;
    const size_t src = (static_cast<size_t>(tok ? t : 0) * num_kv_heads + h) * D;
    T vval{};
    u32x4 kval{};
    if (tok) {
        vval = v[src + d];
        if (d % X == 0) kval = *reinterpret_cast<const u32x4*>(k + src + d);
    }
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
    const int tt = block_size < kTile ? block_size : kTile;  // tokens per tile (8 or 16)
    const int tpb = block_size / tt;
    if (slot < 0 || slot >= static_cast<int64_t>(num_blocks) * block_size) return;
    const int64_t b = slot / block_size;
    const int o = static_cast<int>(slot - b * block_size);
    const int ti = o % tt;
    const int j = ti >> 2, r = ti & 3;
    const size_t tile_base =
        ((static_cast<size_t>(b) * tpb + o / tt) * num_kv_heads + h) * (static_cast<size_t>(tt) * D);
    const int m = d / (16 * E), ee = (d >> 4) % E, i = d & 15;
    v_cache[tile_base + ((((m * (tt / 4) + j) * 16 + i) * E + ee) * 4 + r)] = vval;
    if (d % X == 0)
        *reinterpret_cast<u32x4*>(k_cache + tile_base + ((d / X) * tt + ti) * X) = kval;
}

template <typename T, int D>
hipError_t launch_append(const void* k, const void* v, const int64_t* slots, const int32_t* cow,
                         int num_tokens, void* kc, void* vc, int hkv, int bs, int nb,
                         int32_t* tables, int rows, int cols, const int32_t* upd, int n_upd,
                         const int32_t* lens_in, int32_t* lens_out, int n_lens, hipStream_t st) {
    if (cow && num_tokens > 0) {
        // every copy-on-write copy completes before any token of the step is written
        const hipError_t e = launch_copy_blocks(sizeof(T) == 4 ? 0 : 1, D, bs, hkv, nb, kc, vc,
                                                cow, num_tokens, st);
        if (e != hipSuccess) return e;
    }
    const int extra = (n_upd > n_lens ? n_upd : n_lens);
    const dim3 grid = num_tokens > 0 ? dim3(num_tokens, hkv) : dim3((extra + D - 1) / D, 1);
    if (grid.x == 0) return hipSuccess;
    hipLaunchKernelGGL((append_tokens_kernel<T, D>), grid, dim3(D), 0, st,
                       static_cast<const T*>(k), static_cast<const T*>(v), slots, num_tokens,
                       static_cast<T*>(kc), static_cast<T*>(vc), hkv, bs, nb, tables, rows, cols,
                       upd, n_upd, lens_in, lens_out, n_lens);
    return hipGetLastError();
}

template <typename T, int D>
hipError_t launch_rc(const void* k, const void* v, const int64_t* slots, int num_tokens,
                     void* kc, void* vc, int hkv, int bs, int nb, hipStream_t st) {
    dim3 grid((num_tokens + 15) / 16, hkv);
    hipLaunchKernelGGL((reshape_and_cache_kernel<T, D>), grid, dim3(kWaveSize), 0, st,
                       static_cast<const T*>(k), static_cast<const T*>(v), slots, num_tokens,
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
