// Paged chunked-prefill attention for gfx950.
//
// What is computed: the prompt is processed once, before decoding, all of its
// tokens in one forward pass (ksqn.cn "大模型推理性能优化：PagedAttention与Continuous
// Batching原理与实践", section 2), and a long prompt slows the decoding of the whole
// batch because its attention grows with the square of its length (same page, 5.2
// item 4).  The pages do not say how a prompt is fed; here it is fed a chunk at a
// time, each chunk's keys and values written before it attends.  Generation is
// autoregressive, so a prompt token attends to itself and to every token before it
// (ksqn.cn page, 2.1).  A chunk
// of c tokens of a sequence whose cache holds L tokens (the chunk's own keys and
// values already written, last) puts token i at position L - c + i; it attends to
// cache positions 0 .. L - c + i, through the same block table and K/V layout as
// decode (ksqn.cn page, 2.2).
//
// Work split.  For one KV head, the G query heads of the chunk's tokens form
// (token, head) columns, 16 to a query block: 16 / G consecutive tokens times the G
// heads.  One wavefront folds one query block over the tiles 0 .. (its last
// position) / 16, so the matrix cores see 16 distinct query columns per K/V tile
// instead of decode's G repeated ones.  The tile math (scores, causal mask per
// column, online softmax, PV) is the group tile shared with decode; only the
// visibility limit differs per column.  A workgroup holds four consecutive query
// blocks of one (sequence, KV head); their K/V tiles overlap, so the later waves
// find most of them in L2.  Workgroups are renumbered so that every workgroup of
// one (sequence, KV head) runs on the same XCD (workgroups are dealt to the eight
// XCDs round-robin and each XCD has its own L2), and the blocks with the most
// tiles (the end of a chunk) start first.

#include "kernels_common.h"
#include "pagedkv_internal.h"

namespace pkv {
namespace {

constexpr int kQBlocksPerGroup = 4;  // waves per workgroup
constexpr int kXcds = 8;

template <int D, int G>
__global__ __launch_bounds__(kQBlocksPerGroup * kWave) void prefill_kernel(PrefillArgs a) {
    constexpr int NL = D / 32;     // 16-B loads per lane per tile (K and V)
    constexpr int NG = D / 16;
    constexpr int TB = 16 / G;     // chunk tokens per query block
    constexpr int TILE_U4 = D * 2;
    const int lane = threadIdx.x & (kWave - 1);
    const int wv = threadIdx.x / kWave;

    // workgroup b runs on XCD b % 8: give XCD x the logical groups x * per .. x * per + per - 1
    const int per = (a.num_groups + kXcds - 1) / kXcds;
    const int lg = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (lg >= a.num_groups) return;
    const int qg = a.qgroups - 1 - lg % a.qgroups;  // last query blocks first
    const int sh = lg / a.qgroups;
    const int h = sh % a.num_kv_heads;
    const int s = sh / a.num_kv_heads;
    const int qb = qg * kQBlocksPerGroup + wv;

    const int r0 = a.query_start[s], r1 = a.query_start[s + 1];
    const int c = r1 - r0;
    if (r0 < 0 || r1 > a.num_tokens || c <= 0 || qb * TB >= c) return;
    const int cap = a.max_blocks * a.tiles_per_block * kTile;
    const int L = min(max(a.context_lens[s], 0), cap);
    const int start = L - c;  // position of the chunk's first token (>= 0 for valid input)

    const int j = lane >> 4, i = lane & 15;
    const int tq = qb * TB + i / G;  // chunk token of column i
    const int head = h * G + i % G;  // its query head
    const bool has_row = tq < c;
    const int t_last = min(c - 1, qb * TB + TB - 1);
    const int pmax = start + t_last;  // last position in the block
    using T = uint16_t;
    T* orow = static_cast<T*>(a.out) + (static_cast<size_t>(r0 + tq) * a.num_q_heads + head) * D;
    if (pmax < 0) {  // chunk longer than the cache: no key is visible, rows get zeros
        if (has_row) {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
#pragma unroll
                for (int r = 0; r < 4; ++r) orow[16 * g + 4 * j + r] = 0;
            }
        }
        return;
    }
    // Keys visible to column i: positions < lim.  Columns past the chunk copy the
    // block's last row, and a column before position 0 (invalid input) sees key 0,
    // so that every column's running max is finite; neither is stored as computed.
    const int lim = max(start + (has_row ? tq : t_last), 0) + 1;

    u32x4 q[NL];
    {
        const T* qrow = static_cast<const T*>(a.q) +
                        (static_cast<size_t>(r0 + (has_row ? tq : t_last)) * a.num_q_heads + head) * D;
#pragma unroll
        for (int k = 0; k < NL; ++k) q[k] = *reinterpret_cast<const u32x4*>(qrow + 32 * k + 8 * j);
    }

    const int nt = pmax / kTile + 1;  // tiles to fold
    const int tpb = a.tiles_per_block;
    const int32_t* bt = a.block_tables + static_cast<size_t>(s) * a.max_blocks;
    // Lane k of a window holds the cache position of tile base + k (64 tiles).
    auto window = [&](int base) -> int {
        const int t = base + lane;
        if (t >= nt) return 0;
        int blk = bt[t / tpb];
        blk = static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks) ? blk : 0;
        return (blk * a.num_kv_heads + h) * tpb + t % tpb;
    };
    const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
    const u32x4* vc = static_cast<const u32x4*>(a.v_cache);
    int w_cur = window(0);
    int w_next = nt > kWave ? window(kWave) : 0;  // next window, requested one window ahead
    auto fetch = [&](u32x4 (&kb)[NL], u32x4 (&vb)[NL], int t) {
        if (t > 0 && (t & (kWave - 1)) == 0) {
            w_cur = w_next;
            if (t + kWave < nt) w_next = window(t + kWave);
        }
        const int toff = __builtin_amdgcn_readlane(w_cur, t & (kWave - 1));
        const size_t off = static_cast<size_t>(toff) * TILE_U4;
#pragma unroll
        for (int k = 0; k < NL; ++k) kb[k] = kc[off + lane + k * kWave];
#pragma unroll
        for (int k = 0; k < NL; ++k) vb[k] = vc[off + lane + k * kWave];
    };

    GroupAcc<D> st;
    st.m = kNegInf;
    st.l = 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) st.acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};

    // One tile in flight per wave: wait for everything requested, request the next
    // tile, fold the current one while it travels.
    u32x4 ka[NL], va[NL], kb[NL], vb[NL];
    fetch(ka, va, 0);
    for (int t = 0; t < nt; t += 2) {
        wait_all_loads();
        if (t + 1 < nt) fetch(kb, vb, t + 1);
        group_tile<D, true>(st, q, ka, va, t, lim, L, a.scale_log2e, lane);
        if (t + 1 >= nt) break;
        wait_all_loads();
        if (t + 2 < nt) fetch(ka, va, t + 2);
        group_tile<D, true>(st, q, kb, vb, t + 1, lim, L, a.scale_log2e, lane);
    }

    float l = st.l;
    l += __shfl_xor(l, 16);
    l += __shfl_xor(l, 32);
    if (!has_row) return;
    const bool seen = start + tq >= 0;
    const float inv = seen ? 1.f / l : 0.f;
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        const uint32_t lo = bf16_rne(st.acc[g][0] * inv) | (uint32_t(bf16_rne(st.acc[g][1] * inv)) << 16);
        const uint32_t hi = bf16_rne(st.acc[g][2] * inv) | (uint32_t(bf16_rne(st.acc[g][3] * inv)) << 16);
        *reinterpret_cast<uint2*>(orow + 16 * g + 4 * j) = make_uint2(lo, hi);
    }
}

template <int D>
hipError_t launch_group_size(int group, PrefillArgs& a, hipStream_t st) {
    const dim3 block(kQBlocksPerGroup * kWave);
    const dim3 grid(((a.num_groups + kXcds - 1) / kXcds) * kXcds);
    switch (group) {
        case 1: hipLaunchKernelGGL((prefill_kernel<D, 1>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<D, 2>), grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<D, 4>), grid, block, 0, st, a); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<D, 8>), grid, block, 0, st, a); break;
        case 16: hipLaunchKernelGGL((prefill_kernel<D, 16>), grid, block, 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill(int head_dim, int group, int max_query_len, PrefillArgs& a,
                          hipStream_t stream) {
    if (group < 1 || group > 16 || (16 % group) != 0) return hipErrorInvalidValue;
    const int tb = 16 / group;
    const int qblocks = (max_query_len + tb - 1) / tb;
    a.qgroups = (qblocks + kQBlocksPerGroup - 1) / kQBlocksPerGroup;
    a.num_groups = a.num_seqs * a.num_kv_heads * a.qgroups;
    if (a.num_groups == 0) return hipSuccess;
    if (head_dim == 128) return launch_group_size<128>(group, a, stream);
    if (head_dim == 64) return launch_group_size<64>(group, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
