// Paged chunked-prefill attention for gfx950.
//
// What is computed: the prompt is processed once, before decoding, all of its
// tokens in one forward pass (ksqn.cn "大模型推理性能优化：PagedAttention与Continuous
// Batching原理与实践", section 2), and a long prompt slows the decoding of the whole
// batch because its attention grows with the square of its length (same page, 5.2
// item 4).  The pages do not say how a prompt is fed; here it is fed a chunk at a
// time, each chunk's keys and values written before it attends.  Generation is
// autoregressive, so a prompt token attends to itself and to every token before it
// (ksqn.cn page, 2.1).  A chunk of c tokens of a sequence whose cache holds L tokens
// (the chunk's own keys and values already written, last) puts token i at position
// L - c + i; it attends to cache positions 0 .. L - c + i, through the same block
// table and K/V layout as decode (ksqn.cn page, 2.2).
//
// Work split.  For one KV head, the G query heads of the chunk's tokens form
// (token, head) columns, 16 to a query block: 16 / G consecutive tokens times the G
// heads.  A workgroup of four waves owns 16 consecutive query blocks of one
// (sequence, KV head); wave w folds blocks w, w + 4, w + 8 and w + 12, so that the
// four waves reach the diagonal together.  Keys go by pairs of 16-token tiles: the
// workgroup copies a pair's K and V (16 KiB at D = 128) from the paged cache into
// LDS once, and every wave reads it from there for its 64 columns, so one byte
// fetched from L2 feeds 256 columns.  Two LDS buffers alternate: while the waves
// fold pair p, the registers of every thread carry pair p + 1 in from L2, and one
// barrier per pair hands the buffers over.
//
// Tile math per (query block, pair), all on the matrix cores except the softmax:
//   S^T = K Q^T    v_mfma_f32_16x16x32_bf16, 4 per tile (D = 128): lane (j, i)
//                  gets keys 4j .. 4j + 3 of each tile for column i.
//   O^T += V^T P^T  v_mfma_f32_16x16x32_bf16 over the pair's 32 keys, one per 16
//                  dims.  The contraction runs over keys in the order (tile 0 keys
//                  4j .. 4j + 3, tile 1 keys 4j .. 4j + 3) for the 8 values of lane
//                  (j, i): that is the order in which the S product leaves P in the
//                  lane, and the V tile layout gives the same order from two 8-byte
//                  halves, so neither operand is moved between lanes.
//   l += 1 P^T      the same product with an all-ones A operand: every lane gets its
//                  column's full sum of the rounded weights, no lane reduction.
// The running maximum m of a column moves only when a score exceeds it by more than
// 2^8 (in base-2 units); weights are exp2(score - m) <= 2^8, and the final O / l is
// the same softmax for any m.  So after the first pairs the accumulators are almost
// never rescaled.  P is rounded to bf16 (nearest-even) before both products.
//
// Workgroups are renumbered so that every workgroup of one (sequence, KV head) runs
// on the same XCD (workgroups are dealt to the eight XCDs round-robin and each XCD
// has its own L2), and the query blocks with the most keys (the end of a chunk)
// start first.

#include <type_traits>

#include "kernels_common.h"
#include "pagedkv_internal.h"

namespace pkv {
namespace {

constexpr int kWaves = 4;                  // waves per workgroup
constexpr int kQB = 2;                     // query blocks per wave
constexpr int kThreads = kWaves * kWave;
constexpr int kXcds = 8;
constexpr int kPairKeys = 2 * kTile;
constexpr float kMaxSlack = 8.f;           // base-2 headroom before m moves

typedef __bf16 bf16x2v __attribute__((__vector_size__(2 * sizeof(__bf16))));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const bf16x2v p = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, p);
}

// Maximum over the four lanes 16 apart that hold one column (lanes i, i + 16, i + 32,
// i + 48), with the gfx950 row-swap permutes.
__device__ __forceinline__ float column_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

__device__ __forceinline__ bf16x8 as_bf16x8(uint32_t a, uint32_t b, uint32_t c, uint32_t d) {
    return __builtin_bit_cast(bf16x8, (u32x4){a, b, c, d});
}

template <int D>
struct ColState {
    f32x4 acc[D / 16];  // acc[g][r]: dim 16 g + 4 j + r of column i
    f32x4 lsum;         // every element: the column's sum of weights
    float m;            // the column's reference maximum (base 2)
};

// Fold one pair into one query block.  kEdge: some key of the pair is past the
// block's first causal limit or past the sequence end (per-column masks, zeroed V
// rows past vlim); otherwise every key is visible to every column.
template <int D, bool kEdge>
__device__ __forceinline__ void fold_pair(ColState<D>& st, const u32x4 (&q)[D / 32],
                                          const u32x4 (&k0)[D / 32], const u32x4 (&k1)[D / 32],
                                          const u32x4 (&va)[D / 16], int key0, int lim, int vlim,
                                          float c, int j) {
    constexpr int NL = D / 32;
    f32x4 S0 = {0.f, 0.f, 0.f, 0.f}, S1 = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NL; ++s) {
        S0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k0[s]),
                                                     __builtin_bit_cast(bf16x8, q[s]), S0, 0, 0, 0);
        S1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k1[s]),
                                                     __builtin_bit_cast(bf16x8, q[s]), S1, 0, 0, 0);
    }
    // scores in base-2 units (scale * log2 e folded in)
    float x[8] = {S0[0] * c, S0[1] * c, S0[2] * c, S0[3] * c,
                  S1[0] * c, S1[1] * c, S1[2] * c, S1[3] * c};
    if constexpr (kEdge) {
#pragma unroll
        for (int r = 0; r < 8; ++r) {
            const int key = key0 + (r >> 2) * kTile + 4 * j + (r & 3);
            x[r] = key < lim ? x[r] : kNegInf;
        }
    }
    float mx = fmaxf(fmaxf(fmaxf(x[0], x[1]), fmaxf(x[2], x[3])),
                     fmaxf(fmaxf(x[4], x[5]), fmaxf(x[6], x[7])));
    mx = column_max(mx);
    const bool move = mx > st.m + kMaxSlack;
    if (__ballot(move)) {
        const float mn = move ? mx : st.m;
        const float alpha = fast_exp2(st.m - mn);
#pragma unroll
        for (int g = 0; g < D / 16; ++g) st.acc[g] *= alpha;
        st.lsum *= alpha;
        st.m = mn;
    }
    uint32_t pw[4];
#pragma unroll
    for (int r = 0; r < 4; ++r)
        pw[r] = pack_bf16(fast_exp2(x[2 * r] - st.m), fast_exp2(x[2 * r + 1] - st.m));
    const bf16x8 pB = as_bf16x8(pw[0], pw[1], pw[2], pw[3]);
    uint32_t m00 = 0xffffffffu, m01 = 0xffffffffu, m10 = 0xffffffffu, m11 = 0xffffffffu;
    if constexpr (kEdge) {
        // value rows at or past vlim may hold anything (a zero weight times NaN is NaN)
        const int nv0 = vlim - (key0 + 4 * j), nv1 = nv0 - kTile;
        m00 = (nv0 > 0 ? 0x0000ffffu : 0u) | (nv0 > 1 ? 0xffff0000u : 0u);
        m01 = (nv0 > 2 ? 0x0000ffffu : 0u) | (nv0 > 3 ? 0xffff0000u : 0u);
        m10 = (nv1 > 0 ? 0x0000ffffu : 0u) | (nv1 > 1 ? 0xffff0000u : 0u);
        m11 = (nv1 > 2 ? 0x0000ffffu : 0u) | (nv1 > 3 ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int g = 0; g < D / 16; ++g) {
        bf16x8 vA;
        if constexpr (kEdge)
            vA = as_bf16x8(va[g][0] & m00, va[g][1] & m01, va[g][2] & m10, va[g][3] & m11);
        else
            vA = __builtin_bit_cast(bf16x8, va[g]);
        st.acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, pB, st.acc[g], 0, 0, 0);
    }
    const uint32_t one2 = 0x3f803f80u;  // two bf16 ones
    st.lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(one2, one2, one2, one2), pB,
                                                      st.lsum, 0, 0, 0);
}

template <int D, int G>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
    constexpr int NL = D / 32;                 // 16-B loads per lane per tile (K and V)
    constexpr int NG = D / 16;
    constexpr int TB = 16 / G;                 // chunk tokens per query block
    constexpr int REGION = 2 * D;              // 16-B chunks in one K or V tile
    constexpr int PAIR = 4 * REGION;           // chunks in a pair: K t0, V t0, K t1, V t1
    constexpr int LPT = PAIR / kThreads;       // chunks each thread carries per pair
    // LDS buffer: K t0 | K t1 | V operands.  V operand (g, lane) is 16 bytes: the
    // 8-byte half (g & 1) of V chunk (g / 2) * 64 + lane of tile 0, then the same of
    // tile 1 -- the PV operand of dims 16 g .. for that lane, one read.
    constexpr int VOFF = 2 * REGION;
    static_assert(PAIR % kThreads == 0 && REGION % kWave == 0, "pair split");
    __shared__ u32x4 lds[2][PAIR];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = uni(tid / kWave);

    // workgroup b runs on XCD b % 8: give XCD x the logical groups x * per .. x * per + per - 1
    const int per = (a.num_groups + kXcds - 1) / kXcds;
    const int lg = (blockIdx.x % kXcds) * per + blockIdx.x / kXcds;
    if (lg >= a.num_groups) return;
    const int qg = a.qgroups - 1 - lg % a.qgroups;  // last query blocks first
    const int sh = lg / a.qgroups;
    const int h = sh % a.num_kv_heads;
    const int s = sh / a.num_kv_heads;

    const int r0 = a.query_start[s], r1 = a.query_start[s + 1];
    const int c = r1 - r0;
    const int qb0 = qg * (kWaves * kQB);       // the workgroup's first query block
    if (r0 < 0 || r1 > a.num_tokens || c <= 0 || qb0 * TB >= c) return;  // uniform
    const int cap = a.max_blocks * a.tiles_per_block * kTile;
    const int L = min(max(a.context_lens[s], 0), cap);
    const int start = L - c;  // position of the chunk's first token (>= 0 for valid input)

    const int j = lane >> 4, i = lane & 15;
    // Per query block b of this wave: the columns' causal limits.  Keys visible to
    // column i: positions < lim.  Columns past the chunk copy the block's last row,
    // and a column before position 0 (invalid input) sees key 0, so that every
    // column's maximum is finite; neither is stored as computed.
    int lim[kQB], lim_lo[kQB], lim_hi[kQB], tq[kQB];
    u32x4 q[kQB][NL];
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
        const int tf = (qb0 + b * kWaves + wv) * TB;  // the block's first chunk token
        const int tl = min(c - 1, tf + TB - 1);
        tq[b] = tf + i / G;
        const int row = tq[b] < c ? tq[b] : max(tl, 0);
        lim[b] = max(start + row, 0) + 1;
        lim_lo[b] = tf < c ? max(start + tf, 0) + 1 : 0;
        lim_hi[b] = tf < c ? max(start + tl, 0) + 1 : 0;  // 0: the block is empty
        const uint16_t* qrow = static_cast<const uint16_t*>(a.q) +
                               (static_cast<size_t>(r0 + row) * a.num_q_heads + h * G + i % G) * D;
#pragma unroll
        for (int k = 0; k < NL; ++k) q[b][k] = *reinterpret_cast<const u32x4*>(qrow + 32 * k + 8 * j);
    }
    const float cs = a.scale_log2e;
    // Pairs below p_fast are visible to every column of the wave (all four blocks
    // non-empty); the workgroup folds pairs 0 .. np - 1.
    int p_fast = 1 << 30;
#pragma unroll
    for (int b = 0; b < kQB; ++b) p_fast = min(p_fast, lim_hi[b] == 0 ? 0 : lim_lo[b] / kPairKeys);
    const int t_wg = min(c - 1, (qb0 + kWaves * kQB) * TB - 1);
    const int lim_wg = max(start + t_wg, 0) + 1;
    const int np = (lim_wg + kPairKeys - 1) / kPairKeys;
    const int nt = (lim_wg + kTile - 1) / kTile;  // tiles holding a visible key

    // Cache offsets of tiles, 64 at a time: lane k of a window holds tile base + k.
    const int tpb = a.tiles_per_block;
    const int32_t* bt = a.block_tables + static_cast<size_t>(s) * a.max_blocks;
    auto window = [&](int base) -> int {
        const int t = base + lane;
        if (t >= nt) return 0;  // past the visible tiles: any valid tile, never weighted
        int blk = bt[t / tpb];
        blk = static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks) ? blk : 0;
        return (blk * a.num_kv_heads + h) * tpb + t % tpb;
    };
    const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
    const u32x4* vc = static_cast<const u32x4*>(a.v_cache);
    int w_cur = window(0);
    int w_next = 2 * np > kWave ? window(kWave) : 0;
    u32x4 stg[LPT];
    // Thread tid carries chunks r * 256 + tid of the pair; region (chunk / REGION) is
    // K t0, V t0, K t1, V t1, the same for every lane of a wave.
    auto gload = [&](int p) {
        const int t0 = 2 * p;
        if (t0 > 0 && (t0 & (kWave - 1)) == 0) {
            w_cur = w_next;
            if (t0 + kWave < 2 * np) w_next = window(t0 + kWave);
        }
#pragma unroll
        for (int r = 0; r < LPT; ++r) {
            const int ch = r * kThreads + tid;
            const int reg = uni(ch / REGION);
            const int toff = __builtin_amdgcn_readlane(w_cur, (t0 + (reg >> 1)) & (kWave - 1));
            const u32x4* base = (reg & 1) ? vc : kc;
            stg[r] = base[static_cast<size_t>(toff) * REGION + ch % REGION];
        }
    };
    auto lwrite = [&](int buf) {
#pragma unroll
        for (int r = 0; r < LPT; ++r) {
            const int ch = r * kThreads + tid;
            const int reg = uni(ch / REGION);
            const int o = ch % REGION;
            if ((reg & 1) == 0) {
                lds[buf][(reg >> 1) * REGION + o] = stg[r];
            } else {
                uint2* v2 = reinterpret_cast<uint2*>(&lds[buf][VOFF]);
                const int q0 = (2 * (o / kWave)) * kWave + o % kWave;  // operand (2 mm, lane)
                v2[2 * q0 + (reg >> 1)] = make_uint2(stg[r][0], stg[r][1]);
                v2[2 * (q0 + kWave) + (reg >> 1)] = make_uint2(stg[r][2], stg[r][3]);
            }
        }
    };

    ColState<D> st[kQB];
#pragma unroll
    for (int b = 0; b < kQB; ++b) {
#pragma unroll
        for (int g = 0; g < NG; ++g) st[b].acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
        st[b].lsum = (f32x4){0.f, 0.f, 0.f, 0.f};
        st[b].m = kNegInf;
    }

    gload(0);
    lwrite(0);
    if (np > 1) gload(1);
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    // One pair: read its K and V from LDS, fold it into the wave's blocks, carry the
    // next pair into the other buffer, barrier.
    auto pair_step = [&](int p, auto edge) {
        constexpr bool kEdge = decltype(edge)::value;
        const u32x4* sb = lds[p & 1];
        u32x4 k0[NL], k1[NL], va[NG];
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            k0[k] = sb[k * kWave + lane];
            k1[k] = sb[REGION + k * kWave + lane];
        }
#pragma unroll
        for (int g = 0; g < NG; ++g) va[g] = sb[VOFF + g * kWave + lane];
        const int key0 = p * kPairKeys;
#pragma unroll
        for (int b = 0; b < kQB; ++b) {
            if constexpr (kEdge) {
                // near the diagonal or the sequence end: masks on every block
                if (key0 < lim_hi[b])  // else no key of the pair is visible to the block
                    fold_pair<D, true>(st[b], q[b], k0, k1, va, key0, lim[b], L, cs, j);
            } else {
                fold_pair<D, false>(st[b], q[b], k0, k1, va, key0, 0, 0, cs, j);
            }
        }
        if (p + 1 < np) {
            lwrite((p + 1) & 1);  // that buffer was last read in pair p - 1
            if (p + 2 < np) gload(p + 2);
        }
        // LDS writes done, then the barrier; no fence, so the loads in flight stay in flight
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
    };
    const int pf = min(p_fast, np);
    int p = 0;
    for (; p < pf; ++p) pair_step(p, std::false_type{});
    for (; p < np; ++p) pair_step(p, std::true_type{});

#pragma unroll
    for (int b = 0; b < kQB; ++b) {
        if (lim_hi[b] == 0 || tq[b] >= c) continue;
        uint16_t* orow = static_cast<uint16_t*>(a.out) +
                         (static_cast<size_t>(r0 + tq[b]) * a.num_q_heads + h * G + i % G) * D;
        // a row before position 0 (chunk longer than the cache) has no keys: zeros
        const bool seen = start + tq[b] >= 0;
        const float inv = 1.f / st[b].lsum[0];
#pragma unroll
        for (int g = 0; g < NG; ++g) {
            uint32_t lo = bf16_rne(st[b].acc[g][0] * inv) |
                          (uint32_t(bf16_rne(st[b].acc[g][1] * inv)) << 16);
            uint32_t hi = bf16_rne(st[b].acc[g][2] * inv) |
                          (uint32_t(bf16_rne(st[b].acc[g][3] * inv)) << 16);
            if (!seen) lo = hi = 0u;
            *reinterpret_cast<uint2*>(orow + 16 * g + 4 * j) = make_uint2(lo, hi);
        }
    }
}

template <int D>
hipError_t launch_group_size(int group, PrefillArgs& a, hipStream_t st) {
    const dim3 block(kThreads);
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
    a.qgroups = (qblocks + kWaves * kQB - 1) / (kWaves * kQB);
    a.num_groups = a.num_seqs * a.num_kv_heads * a.qgroups;
    if (a.num_groups == 0) return hipSuccess;
    if (head_dim == 128) return launch_group_size<128>(group, a, stream);
    if (head_dim == 64) return launch_group_size<64>(group, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
