// Read-bandwidth probe with the decode kernel's access pattern (declared in
// include/pagedkv_probe.h): eight-wave workgroups, each step one 32 KiB chunk of K
// and one of V, a wave reading its 4 KiB slice of each with one 16-byte load per
// lane per KiB.  Built as its own library; the paged-attention path never calls it.

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "pagedkv_probe.h"

namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));

constexpr int kWaves = 8;                      // waves per workgroup (one per KV head)
constexpr int kSliceU4 = 4096 / 16;            // one wave's slice of a chunk, 16-B units
constexpr int kChunkU4 = kWaves * kSliceU4;    // a 32 KiB chunk
constexpr int kLoads = kSliceU4 / 64;          // 16-B loads per lane per slice (4)

struct Tile {
    u32x4 k[kLoads], v[kLoads];
};

template <bool NT>
__device__ __forceinline__ void fetch(Tile& t, const u32x4* k, const u32x4* v, int64_t chunk,
                                      int wave, int lane) {
    const u32x4* kp = k + chunk * kChunkU4 + wave * kSliceU4 + lane;
    const u32x4* vp = v + chunk * kChunkU4 + wave * kSliceU4 + lane;
#pragma unroll
    for (int s = 0; s < kLoads; ++s) t.k[s] = NT ? __builtin_nontemporal_load(kp + 64 * s) : kp[64 * s];
#pragma unroll
    for (int s = 0; s < kLoads; ++s) t.v[s] = NT ? __builtin_nontemporal_load(vp + 64 * s) : vp[64 * s];
}

__device__ __forceinline__ unsigned fold(const Tile& t) {
    unsigned x = 0;
#pragma unroll
    for (int s = 0; s < kLoads; ++s) x ^= t.k[s][0] ^ t.k[s][1] ^ t.k[s][2] ^ t.k[s][3] ^
                                          t.v[s][0] ^ t.v[s][1] ^ t.v[s][2] ^ t.v[s][3];
    return x;
}

template <bool NT, int InFlight>
__global__ __launch_bounds__(64 * kWaves) void gather_read(const u32x4* __restrict__ k,
                                                           const u32x4* __restrict__ v,
                                                           int64_t num_chunks,
                                                           const int32_t* __restrict__ order,
                                                           int chunks_per_group,
                                                           uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int32_t* ord = order + static_cast<int64_t>(blockIdx.x) * chunks_per_group;
    auto chunk_of = [&](int i) -> int64_t {
        const int64_t c = ord[i];
        return (c >= 0 && c < num_chunks) ? c : 0;
    };
    unsigned acc = 0;
    if constexpr (InFlight == 1) {
        for (int i = 0; i < chunks_per_group; ++i) {
            Tile t;
            fetch<NT>(t, k, v, chunk_of(i), wave, lane);
            acc ^= fold(t);  // the fold waits for this tile before the next is requested
        }
    } else {
        Tile a, b;
        int i = 0;
        if (chunks_per_group > 0) fetch<NT>(a, k, v, chunk_of(0), wave, lane);
        for (; i + 2 < chunks_per_group; i += 2) {
            fetch<NT>(b, k, v, chunk_of(i + 1), wave, lane);
            acc ^= fold(a);
            fetch<NT>(a, k, v, chunk_of(i + 2), wave, lane);
            acc ^= fold(b);
        }
        if (i + 1 < chunks_per_group) {
            fetch<NT>(b, k, v, chunk_of(i + 1), wave, lane);
            acc ^= fold(a);
            acc ^= fold(b);
        } else if (i < chunks_per_group) {
            acc ^= fold(a);
        }
    }
    // one value per wave
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if (lane == 0) sink[blockIdx.x * kWaves + wave] = acc;
}

// The same read pattern through raw buffer loads with explicit cache-policy bits
// (gfx950: bit 0 sc0, bit 1 nt, bit 4 sc1), one tile in flight per wave.
constexpr int kBufferRsrcWord3 = 0x00020000;  // 32-bit data format, no swizzle

template <int Policy>
__global__ __launch_bounds__(64 * kWaves) void gather_read_policy(const u32x4* __restrict__ k,
                                                                  const u32x4* __restrict__ v,
                                                                  int64_t num_chunks,
                                                                  const int32_t* __restrict__ order,
                                                                  int chunks_per_group,
                                                                  uint32_t* __restrict__ sink) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) >> 6);
    const int32_t* ord = order + static_cast<int64_t>(blockIdx.x) * chunks_per_group;
    const int bytes = static_cast<int>(num_chunks * kChunkU4 * 16);  // checked < 2^31 by the host
    const __amdgpu_buffer_rsrc_t kr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4*>(k), static_cast<short>(0), bytes, kBufferRsrcWord3);
    const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<u32x4*>(v), static_cast<short>(0), bytes, kBufferRsrcWord3);
    unsigned acc = 0;
    for (int i = 0; i < chunks_per_group; ++i) {
        int64_t c = ord[i];
        c = (c >= 0 && c < num_chunks) ? c : 0;
        const int base = static_cast<int>((c * kChunkU4 + wave * kSliceU4 + lane) * 16);
        Tile t;
#pragma unroll
        for (int s = 0; s < kLoads; ++s)
            t.k[s] = __builtin_amdgcn_raw_buffer_load_b128(kr, base + s * 1024, 0, Policy);
#pragma unroll
        for (int s = 0; s < kLoads; ++s)
            t.v[s] = __builtin_amdgcn_raw_buffer_load_b128(vr, base + s * 1024, 0, Policy);
        acc ^= fold(t);
    }
    for (int o = 32; o > 0; o >>= 1) acc ^= __shfl_xor(acc, o);
    if (lane == 0) sink[blockIdx.x * kWaves + wave] = acc;
}

}  // namespace

extern "C" int32_t pa_probe_gather_read_policy(const void* k, const void* v, int64_t num_chunks,
                                               const int32_t* order, int32_t num_groups,
                                               int32_t chunks_per_group, uint32_t* sink,
                                               int32_t cache_policy, void* stream) {
    if (!k || !v || !order || !sink || num_chunks <= 0 || num_groups <= 0 ||
        chunks_per_group < 0 || num_chunks * 32768 >= (int64_t(1) << 31) ||
        (reinterpret_cast<uintptr_t>(k) & 15) || (reinterpret_cast<uintptr_t>(v) & 15))
        return 1;
    const dim3 grid(num_groups), block(64 * kWaves);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4* kk = static_cast<const u32x4*>(k);
    const u32x4* vv = static_cast<const u32x4*>(v);
#define PA_POLICY(P)                                                                          \
    case P:                                                                                   \
        hipLaunchKernelGGL((gather_read_policy<P>), grid, block, 0, st, kk, vv, num_chunks,  \
                           order, chunks_per_group, sink);                                    \
        break;
    switch (cache_policy) {
        PA_POLICY(0) PA_POLICY(1) PA_POLICY(2) PA_POLICY(3)
        PA_POLICY(16) PA_POLICY(17) PA_POLICY(18) PA_POLICY(19)
        default: return 1;
    }
#undef PA_POLICY
    return hipGetLastError() == hipSuccess ? 0 : 5;
}

extern "C" int32_t pa_probe_gather_read(const void* k, const void* v, int64_t num_chunks,
                                        const int32_t* order, int32_t num_groups,
                                        int32_t chunks_per_group, uint32_t* sink,
                                        int32_t nontemporal, int32_t in_flight, void* stream) {
    if (!k || !v || !order || !sink || num_chunks <= 0 || num_groups <= 0 ||
        chunks_per_group < 0 || (in_flight != 1 && in_flight != 2) ||
        (reinterpret_cast<uintptr_t>(k) & 15) || (reinterpret_cast<uintptr_t>(v) & 15))
        return 1;
    const dim3 grid(num_groups), block(64 * kWaves);
    hipStream_t st = static_cast<hipStream_t>(stream);
    const u32x4* kk = static_cast<const u32x4*>(k);
    const u32x4* vv = static_cast<const u32x4*>(v);
    if (nontemporal) {
        if (in_flight == 1)
            hipLaunchKernelGGL((gather_read<true, 1>), grid, block, 0, st, kk, vv, num_chunks, order, chunks_per_group, sink);
        else
            hipLaunchKernelGGL((gather_read<true, 2>), grid, block, 0, st, kk, vv, num_chunks, order, chunks_per_group, sink);
    } else {
        if (in_flight == 1)
            hipLaunchKernelGGL((gather_read<false, 1>), grid, block, 0, st, kk, vv, num_chunks, order, chunks_per_group, sink);
        else
            hipLaunchKernelGGL((gather_read<false, 2>), grid, block, 0, st, kk, vv, num_chunks, order, chunks_per_group, sink);
    }
    return hipGetLastError() == hipSuccess ? 0 : 5;
}
