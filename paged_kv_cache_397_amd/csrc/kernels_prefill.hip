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
// heads.  A workgroup of four waves owns 8 consecutive query blocks of one
// (sequence, KV head); wave w folds blocks w and w + 4, so that the four waves reach
// the diagonal together.  Keys go by pairs of 16-token tiles: the workgroup copies
// a pair's K and V (16 KiB at D = 128) straight from the paged cache into LDS once
// (global_load_lds), and every wave reads it from there for its 32 columns, so one
// byte fetched from L2 feeds 128 columns.  Four LDS buffers hold pairs p .. p + 3:
// the copies run three pairs ahead, one barrier per pair hands a buffer over, and
// the matrix cores compute the scores of pair p + 1 while pair p is folded.
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
// has its own L2), the (sequence, KV head) pairs are dealt to the XCDs round-robin
// (an even mix of lengths per XCD), the longest sequences start first, and within a
// sequence the query blocks with the most keys (the end of a chunk) start first.

#include <climits>
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
constexpr int kStages = 4;                 // LDS buffers: pairs p .. p + 3 resident or in flight

typedef __bf16 bf16x2v __attribute__((__vector_size__(2 * sizeof(__bf16))));

__device__ __forceinline__ uint32_t pack_bf16(float lo, float hi) {
    const bf16x2v p = {static_cast<__bf16>(lo), static_cast<__bf16>(hi)};
    return __builtin_bit_cast(uint32_t, p);
}

// IEEE maximum (NaN-propagating): gfx950 has it as one instruction that needs no
// quieting of its inputs, unlike fmaxf.
__device__ __forceinline__ float vmax(float a, float b) { return __builtin_elementwise_maximum(a, b); }

// Maximum over the four lanes 16 apart that hold one column (lanes i, i + 16, i + 32,
// i + 48), with the gfx950 row-swap permutes.
__device__ __forceinline__ float column_max(float x) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    x = vmax(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false,
                                                    false);
    return vmax(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// Byte address of an LDS object, as the ds_* instructions take it.
template <typename T>
__device__ __forceinline__ uint32_t lds_addr(const T* p) {
    return static_cast<uint32_t>(
        reinterpret_cast<size_t>((const char __attribute__((address_space(3)))*)p));
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

// Scores of one pair for the wave's NB query blocks (four independent MFMA chains
// for NB = 2): S0 for tile 0, S1 for tile 1.  Masked: only the blocks whose bit is
// set in `act` (uniform) are computed; the others are left as they are.
template <int D, int NB, bool Masked = false>
__device__ __forceinline__ void pair_scores(f32x4 (&S0)[NB], f32x4 (&S1)[NB],
                                            const u32x4 (&q)[NB][D / 32],
                                            const u32x4 (&k0)[D / 32], const u32x4 (&k1)[D / 32],
                                            uint32_t act = ~0u) {
#pragma unroll
    for (int b = 0; b < NB; ++b) S0[b] = S1[b] = (f32x4){0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < D / 32; ++s) {
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (Masked && !((act >> b) & 1u)) continue;
            S0[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k0[s]),
                                                            __builtin_bit_cast(bf16x8, q[b][s]),
                                                            S0[b], 0, 0, 0);
            S1[b] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, k1[s]),
                                                            __builtin_bit_cast(bf16x8, q[b][s]),
                                                            S1[b], 0, 0, 0);
        }
    }
}

// Folding one pair's scores into the wave's NB query blocks, in pieces that run on
// different units so that one pair's vector work can overlap another pair's matrix
// work:
//   pair_max (VALU): scores to base-2 units with masks, each column's maximum, and
//     whether any column's reference maximum has to move;
//   rescale (VALU, rare): move the reference maxima, rescale the accumulators;
//   pair_weights (VALU): the weights exp2(score - m), rounded to bf16;
//   pair_pv (MFMA): O^T += V^T P^T and l += 1 P^T.
// kEdge: some key of the pair may be past a column's causal limit or past the
// sequence end: per-column masks, and V rows at or past vlim zeroed (they may hold
// anything, and a zero weight times NaN is NaN).  Otherwise every key is visible to
// every column.  c >= 0 (scale * log2 e).
template <int D, int NB, bool kEdge, bool Masked = false>
__device__ __forceinline__ bool pair_max(const ColState<D> (&st)[NB], float (&x)[NB][8],
                                         float (&mx)[NB], const f32x4 (&S0)[NB],
                                         const f32x4 (&S1)[NB], int key0, const int (&lim)[NB],
                                         float c, int j, uint32_t act = ~0u) {
    bool any = false;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if (Masked && !((act >> b) & 1u)) {
            mx[b] = kNegInf;  // a block that sees no key of the pair: nothing moves
            continue;
        }
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            x[b][r] = S0[b][r];
            x[b][4 + r] = S1[b][r];
        }
        if constexpr (kEdge) {
#pragma unroll
            for (int r = 0; r < 8; ++r) {
                const int key = key0 + (r >> 2) * kTile + 4 * j + (r & 3);
                x[b][r] = key < lim[b] ? x[b][r] : kNegInf;
            }
        }
        float m8 = vmax(vmax(vmax(x[b][0], x[b][1]), vmax(x[b][2], x[b][3])),
                        vmax(vmax(x[b][4], x[b][5]), vmax(x[b][6], x[b][7])));
        mx[b] = column_max(m8) * c;
        any |= mx[b] > st[b].m + kMaxSlack;
    }
    return any;
}

template <int D, int NB>
__device__ __forceinline__ void rescale(ColState<D> (&st)[NB], const float (&mx)[NB]) {
    constexpr int NG = D / 16;
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        const float mn = mx[b] > st[b].m + kMaxSlack ? mx[b] : st[b].m;
        const float alpha = fast_exp2(st[b].m - mn);
#pragma unroll
        for (int g = 0; g < NG; ++g) st[b].acc[g] *= alpha;
        st[b].lsum *= alpha;
        st[b].m = mn;
    }
}

template <int D, int NB, bool Masked = false>
__device__ __forceinline__ void pair_weights(bf16x8 (&pB)[NB], const ColState<D> (&st)[NB],
                                             const float (&x)[NB][8], float c, uint32_t act = ~0u) {
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if (Masked && !((act >> b) & 1u)) continue;
        uint32_t pw[4];
#pragma unroll
        for (int r = 0; r < 4; ++r)
            pw[r] = pack_bf16(fast_exp2(__builtin_fmaf(x[b][2 * r], c, -st[b].m)),
                              fast_exp2(__builtin_fmaf(x[b][2 * r + 1], c, -st[b].m)));
        pB[b] = as_bf16x8(pw[0], pw[1], pw[2], pw[3]);
    }
}

template <int D, int NB, bool kEdge, bool Masked = false>
__device__ __forceinline__ void pair_pv(ColState<D> (&st)[NB], const bf16x8 (&pB)[NB],
                                        u32x4 (&va)[D / 16], int key0, int vlim, int j,
                                        uint32_t act = ~0u) {
    constexpr int NG = D / 16;
    // the V operands were read by inline asm the compiler does not track: wait here
#pragma unroll
    for (int g = 0; g < NG; ++g) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(va[g]));
    uint32_t m00 = 0xffffffffu, m01 = 0xffffffffu, m10 = 0xffffffffu, m11 = 0xffffffffu;
    if constexpr (kEdge) {
        const int nv0 = vlim - (key0 + 4 * j), nv1 = nv0 - kTile;
        m00 = (nv0 > 0 ? 0x0000ffffu : 0u) | (nv0 > 1 ? 0xffff0000u : 0u);
        m01 = (nv0 > 2 ? 0x0000ffffu : 0u) | (nv0 > 3 ? 0xffff0000u : 0u);
        m10 = (nv1 > 0 ? 0x0000ffffu : 0u) | (nv1 > 1 ? 0xffff0000u : 0u);
        m11 = (nv1 > 2 ? 0x0000ffffu : 0u) | (nv1 > 3 ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int g = 0; g < NG; ++g) {
        bf16x8 vA;
        if constexpr (kEdge)
            vA = as_bf16x8(va[g][0] & m00, va[g][1] & m01, va[g][2] & m10, va[g][3] & m11);
        else
            vA = __builtin_bit_cast(bf16x8, va[g]);
#pragma unroll
        for (int b = 0; b < NB; ++b) {
            if (Masked && !((act >> b) & 1u)) continue;
            st[b].acc[g] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(vA, pB[b], st[b].acc[g], 0, 0, 0);
        }
    }
    const uint32_t one2 = 0x3f803f80u;  // two bf16 ones
#pragma unroll
    for (int b = 0; b < NB; ++b) {
        if (Masked && !((act >> b) & 1u)) continue;
        st[b].lsum = __builtin_amdgcn_mfma_f32_16x16x32_bf16(as_bf16x8(one2, one2, one2, one2),
                                                             pB[b], st[b].lsum, 0, 0, 0);
    }
}

// Scheduling hints: within the current region, alternate n_mfma groups of one matrix
// instruction with `valu` vector instructions each, so that one pair's softmax runs
// on the vector ALUs while the matrix cores work on another pair (the compiler would
// otherwise cluster each kind).
template <int NMfma, int Valu>
__device__ __forceinline__ void interleave_mfma_valu() {
#pragma unroll
    for (int k = 0; k < NMfma; ++k) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);     // one MFMA
        __builtin_amdgcn_sched_group_barrier(0x002, Valu, 0);  // then VALU instructions
    }
}

// Half: blocks of 8 tokens; a 16-token tile is copied from two blocks (tokens 0..7
// of K and key quads 0..1 of V from the first, the rest from the second), so LDS
// holds the same 16-token tiles either way.
template <int D, int G, bool Half>
__global__ __launch_bounds__(kThreads) __attribute__((amdgpu_waves_per_eu(2, 2)))
void prefill_kernel(PrefillArgs a) {
    constexpr int NL = D / 32;                 // 16-B loads per lane per tile (K and V)
    constexpr int NG = D / 16;
    constexpr int TB = 16 / G;                 // chunk tokens per query block
    constexpr int REGION = 2 * D;              // 16-B chunks in one K or V tile
    constexpr int PAIR = 4 * REGION;           // chunks in a pair: K t0, V t0, K t1, V t1
    constexpr int LPT = PAIR / kThreads;       // chunks each thread copies per pair
    static_assert(PAIR % kThreads == 0 && REGION % kWave == 0 && kThreads % REGION == 0 &&
                      (kStages & (kStages - 1)) == 0, "pair split");
    static_assert((kStages - 2) * LPT < 16, "vmcnt immediate");
    __shared__ u32x4 lds[kStages][PAIR];

    const int tid = threadIdx.x;
    const int lane = tid & (kWave - 1);
    const int wv = uni(tid / kWave);

    // Workgroup b runs on XCD x = b % 8.  XCD x takes the (sequence, KV head) pairs
    // sh = s Hkv + h with sh = x (mod 8), all query groups of one pair in a row (they
    // share its K/V in that XCD's L2), the last query groups (most keys) first.
    // Dealing the pairs round-robin gives every XCD a similar mix of sequence lengths.
    const int xcd = blockIdx.x % kXcds, k = blockIdx.x / kXcds;
    const int Hkv = a.num_kv_heads;
    const int nsh = a.num_seqs * Hkv;
    if (k >= ((nsh - xcd + kXcds - 1) / kXcds) * a.qgroups) return;
    const int qg = a.qgroups - 1 - k % a.qgroups;
    int jj = k / a.qgroups;  // this workgroup's (sequence, KV head) among the XCD's
    int s, h, r0, r1, Lraw;
    if (a.num_seqs <= kWave) {
        // Longest sequences first (ties: lower index), so that the longest workgroups
        // do not start last.  Lane t ranks sequence t by cache length; a forward
        // permute gives lane r the sequence of rank r; lane r counts that sequence's
        // heads on this XCD (sequence s has heads h = (x - s Hkv) mod 8, + 8, ...);
        // a scan over the lanes finds the rank whose heads hold entry jj.
        const int lane0 = threadIdx.x & (kWave - 1);
        const bool is_seq = lane0 < a.num_seqs;
        const int Ls = is_seq ? a.context_lens[lane0] : INT_MIN;
        const int qa = is_seq ? a.query_start[lane0] : 0;
        const int qb = is_seq ? a.query_start[lane0 + 1] : 0;
        int rank = is_seq ? 0 : lane0;  // lanes past the batch keep distinct ranks >= S
        for (int t = 0; t < a.num_seqs; ++t) {
            const int Lt = __builtin_amdgcn_readlane(Ls, t);
            rank += is_seq && ((Lt > Ls) || (Lt == Ls && t < lane0));
        }
        const int sr = __builtin_amdgcn_ds_permute(rank * 4, lane0);  // sequence of rank lane0
        const int h0 = (xcd - sr * Hkv) & (kXcds - 1);
        const int cnt = is_seq && h0 < Hkv ? (Hkv - 1 - h0) / kXcds + 1 : 0;
        const int incl = wave_inclusive_scan(cnt, lane0);
        const int r = uni(__builtin_ffsll(__ballot(incl > jj)) - 1);  // exists: jj < heads on XCD
        s = __builtin_amdgcn_readlane(sr, r);
        h = __builtin_amdgcn_readlane(h0, r) +
            kXcds * (jj - (__builtin_amdgcn_readlane(incl, r) - __builtin_amdgcn_readlane(cnt, r)));
        r0 = __builtin_amdgcn_readlane(qa, s);
        r1 = __builtin_amdgcn_readlane(qb, s);
        Lraw = __builtin_amdgcn_readlane(Ls, s);
    } else {
        const int sh = xcd + kXcds * jj;
        h = sh % Hkv;
        s = sh / Hkv;
        r0 = a.query_start[s];
        r1 = a.query_start[s + 1];
        Lraw = a.context_lens[s];
    }

    const int c = r1 - r0;
    const int qb0 = qg * (kWaves * kQB);       // the workgroup's first query block
    if (r0 < 0 || r1 > a.num_tokens || c <= 0 || qb0 * TB >= c) return;  // uniform
    const int cap = a.max_blocks * a.block_size;
    const int L = min(max(Lraw, 0), cap);
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
    // The pair maximum is taken on raw scores and scaled after, and masked keys carry
    // a raw -inf that the scaling keeps -inf, which needs c > 0.  For a negative scale,
    // negate q (exact in bf16) and use -c, the same products.  For a zero scale (every
    // visible key weighs the same; -inf * 0 would be NaN) use the smallest normal
    // float: a score under 2^26 in magnitude times it is under 2^-100, whose exp2 is 1
    // in fp32, as for 0, and a masked key's weight stays 0.
    float cs = a.scale_log2e;
    if (cs < 0.f) {
        cs = -cs;
#pragma unroll
        for (int b = 0; b < kQB; ++b) {
#pragma unroll
            for (int k = 0; k < NL; ++k) q[b][k] ^= 0x80008000u;
        }
    }
    if (!(cs > 0.f)) cs = __FLT_MIN__;
    // Pairs below p_fast are visible to every column of the wave (both blocks
    // non-empty); the workgroup folds pairs 0 .. np - 1.
    int p_fast = 1 << 30;
#pragma unroll
    for (int b = 0; b < kQB; ++b) p_fast = min(p_fast, lim_hi[b] == 0 ? 0 : lim_lo[b] / kPairKeys);
    const int t_wg = min(c - 1, (qb0 + kWaves * kQB) * TB - 1);
    const int lim_wg = max(start + t_wg, 0) + 1;
    const int np = (lim_wg + kPairKeys - 1) / kPairKeys;
    const int nt = (lim_wg + kTile - 1) / kTile;  // tiles holding a visible key

    // Block ids of tiles, WT tiles at a time: lane k of a window holds the block of
    // tile base + k (Half: table entry 2 base + k, the two blocks of tiles base ..
    // base + 31).  Window 0 is read here; window w + 1 is copied by wave 0 into an
    // LDS ring when window w comes into use, WT / 2 pairs before it is needed, so its
    // copy is covered by the pair loop's waits and barriers like the K/V copies.
    constexpr int WT = Half ? kWave / 2 : kWave;
    const int tpb = a.tiles_per_block;
    const int32_t* bt = a.block_tables + static_cast<size_t>(s) * a.max_blocks;
    const int last_entry = max((L - 1) >> 3, 0);  // Half: the sequence's last block
    __shared__ int win_lds[2][kWave];
    auto win_src = [&](int base) -> const int32_t* {
        if constexpr (Half) {
            // the second block of a tile the sequence ends before reads the first again
            const int e = 2 * base + lane;
            return bt + (e < 2 * nt ? min(e, last_entry) : 0);
        } else {
            const int t = base + lane;
            return bt + (t < nt ? t / tpb : 0);  // past the visible tiles: any valid tile, never weighted
        }
    };
    auto copy_window = [&](int base) {
        if (wv == 0)
            __builtin_amdgcn_global_load_lds(
                (const void __attribute__((address_space(1)))*)win_src(base),
                (void __attribute__((address_space(3)))*)&win_lds[(base / WT) & 1][0], 4, 0, 0);
    };
    // lane's tile base + lane (Half: lane's block): block id -> the tile's index in
    // the cache (once per window)
    auto tile_offset = [&](int blk, int base) -> int {
        blk = static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks) ? blk : 0;
        if constexpr (Half) return blk * a.num_kv_heads + h;
        return (blk * tpb + (base + lane) % tpb) * a.num_kv_heads + h;
    };
    const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
    const u32x4* vc = static_cast<const u32x4*>(a.v_cache);
    int w_cur = tile_offset(*win_src(0), 0);
    if (2 * np > WT) copy_window(WT);
    // Thread tid copies chunks r * 256 + tid of the pair straight from the cache into
    // LDS (global_load_lds: lane l of a wave lands 16 bytes at the wave's LDS base +
    // 16 l); region (chunk / REGION) is K t0, V t0, K t1, V t1, the same for every
    // lane of a wave.  The compiler does not order these copies against LDS reads:
    // the pair loop waits for them explicitly (vmcnt) before its barrier.
    auto issue = [&](int p) {
        const int t0 = 2 * p;
        if (t0 > 0 && (t0 & (WT - 1)) == 0) {
            int raw;
            asm volatile("ds_read_b32 %0, %1\n\ts_waitcnt lgkmcnt(0)"
                         : "=v"(raw) : "v"(lds_addr(&win_lds[(t0 / WT) & 1][lane])));
            w_cur = tile_offset(raw, t0);
            if (t0 + WT < 2 * np) copy_window(t0 + WT);
        }
        u32x4* stage = lds[p & (kStages - 1)];
#pragma unroll
        for (int r = 0; r < LPT; ++r) {
            // this wave's 64 chunks of copy r: rw .. rw + 63, all in one region
            const int rw = r * kThreads + wv * kWave;
            const int reg = r * (kThreads / REGION) + (wv * kWave) / REGION;
            if constexpr (Half) {
                // chunk cidx of the 16-token tile: K (token cidx % 16, dims chunk cidx / 16)
                // sits in block token / 8; V (quad (cidx / 16) % 4) in block quad / 2
                constexpr int HALF = REGION / 2;
                const int t = t0 + (reg >> 1);
                const int toffA = __builtin_amdgcn_readlane(w_cur, (2 * t) & (kWave - 1));
                const int toffB = __builtin_amdgcn_readlane(w_cur, (2 * t + 1) & (kWave - 1));
                const int cidx = (rw & (REGION - 1)) + lane;
                const u32x4* src;
                if (reg & 1) {
                    const int jq = (cidx >> 4) & 3;
                    src = vc + static_cast<size_t>(jq < 2 ? toffA : toffB) * HALF +
                          ((cidx >> 6) * 2 + (jq & 1)) * 16 + (cidx & 15);
                } else {
                    const int tok = cidx & 15;
                    src = kc + static_cast<size_t>(tok < 8 ? toffA : toffB) * HALF +
                          (cidx >> 4) * 8 + (tok & 7);
                }
                __builtin_amdgcn_global_load_lds((const void __attribute__((address_space(1)))*)src,
                                                 (void __attribute__((address_space(3)))*)(stage + rw),
                                                 16, 0, 0);
            } else {
                const int toff = __builtin_amdgcn_readlane(w_cur, (t0 + (reg >> 1)) & (kWave - 1));
                const u32x4* src = ((reg & 1) ? vc : kc) + static_cast<size_t>(toff) * REGION;
                __builtin_amdgcn_global_load_lds(
                    (const void __attribute__((address_space(1)))*)(src + (rw & (REGION - 1)) + lane),
                    (void __attribute__((address_space(3)))*)(stage + rw), 16, 0, 0);
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

    for (int i = 0; i < kStages - 1 && i < np; ++i) issue(i);

    // LDS reads by inline asm: the compiler would make every LDS read wait for all
    // copies in flight (it cannot tell the buffers apart), which would drain the
    // pipeline each pair.  LDS reads complete in order; the waits below rely on it.
    typedef unsigned u32x2 __attribute__((ext_vector_type(2)));
    auto read_k = [&](int p, u32x4 (&k0)[NL], u32x4 (&k1)[NL]) {
        const uint32_t laddr = lds_addr(lds[p & (kStages - 1)]) + lane * 16;
#pragma unroll
        for (int k = 0; k < NL; ++k) {
            asm volatile("ds_read_b128 %0, %1 offset:%2" : "=v"(k0[k]) : "v"(laddr), "i"(k * kWave * 16));
            asm volatile("ds_read_b128 %0, %1 offset:%2"
                         : "=v"(k1[k]) : "v"(laddr), "i"(2 * REGION * 16 + k * kWave * 16));
        }
    };
    // PV operand of dims 16 g = 32 mm + 16 e: the 8-byte half e of V chunk mm * 64 + lane
    // of tile 0, then the same of tile 1, read into the operand's halves (fold_pv
    // waits for them).
    auto read_v = [&](int p, u32x4 (&va)[NG]) {
        const uint32_t laddr = lds_addr(lds[p & (kStages - 1)]) + lane * 16;
#pragma unroll
        for (int mm = 0; mm < NL; ++mm) {
#pragma unroll
            for (int e = 0; e < 2; ++e) {
                u32x2 lo, hi;
                asm volatile("ds_read_b64 %0, %1 offset:%2"
                             : "=v"(lo) : "v"(laddr), "i"(REGION * 16 + mm * kWave * 16 + 8 * e));
                asm volatile("ds_read_b64 %0, %1 offset:%2"
                             : "=v"(hi) : "v"(laddr), "i"(3 * REGION * 16 + mm * kWave * 16 + 8 * e));
                va[2 * mm + e] = (u32x4){lo.x, lo.y, hi.x, hi.y};
            }
        }
    };

    // Software pipeline.  Step p folds pair p and prepares pair p + 1 in two phases,
    // each pairing one unit's work on one pair with the other unit's on the other:
    //   A: the weights of pair p (vector ALUs)  |  the scores of pair p + 1 (matrix)
    //   B: O += V P of pair p (matrix)          |  the maxima of pair p + 1 (vector)
    // then, rarely, pair p + 1's rescale.  Pair 0's scores and maxima come first:
    // wait for its copies (later pairs' may stay in flight).
    // Pairs below p_fast are unmasked; the last pair is always masked (pf <= np - 1).
    const int pf = min(p_fast, np - 1);
    // Blocks that see a key of pair p (uniform): block b's last such pair is
    // (lim_hi[b] - 1) / 32; an empty block (lim_hi = 0) sees none.
    int last_pair[kQB];
#pragma unroll
    for (int b = 0; b < kQB; ++b) last_pair[b] = lim_hi[b] == 0 ? -1 : (lim_hi[b] - 1) / kPairKeys;
    auto active_at = [&](int pp) -> uint32_t {
        uint32_t m = 0;
#pragma unroll
        for (int b = 0; b < kQB; ++b) m |= (pp <= last_pair[b] ? 1u : 0u) << b;
        return uni(static_cast<int>(m));
    };
    f32x4 S0[kQB], S1[kQB];
    float x[kQB][8];
    if (np >= kStages - 1)
        __builtin_amdgcn_s_waitcnt(0x0F70 | ((kStages - 2) * LPT));
    else
        __builtin_amdgcn_s_waitcnt(0x0F70);
    asm volatile("s_barrier" ::: "memory");
    {
        u32x4 k0[NL], k1[NL];
        read_k(0, k0, k1);
#pragma unroll
        for (int k = 0; k < NL; ++k) asm volatile("s_waitcnt lgkmcnt(0)" : "+v"(k0[k]), "+v"(k1[k]));
        pair_scores<D, kQB>(S0, S1, q, k0, k1);
        float mx[kQB];
        const bool any = pf == 0 ? pair_max<D, kQB, true>(st, x, mx, S0, S1, 0, lim, cs, j)
                                 : pair_max<D, kQB, false>(st, x, mx, S0, S1, 0, lim, cs, j);
        if (__ballot(any)) rescale<D, kQB>(st, mx);
    }

    // Step p: wait for pair p + 1's copies and barrier (pair p - 1's buffer is then
    // free: its K was read in step p - 1, its V in step p - 1), start the copy of pair
    // p + 3 into it, read K of pair p + 1 and V of pair p, then phases A and B.
    // kEdge: pair p is masked; kEdgeNext: pair p + 1 is.
    auto pair_step = [&](int p, auto edge, auto edge_next, auto next) {
        constexpr bool kEdge = decltype(edge)::value;
        constexpr bool kEdgeNext = decltype(edge_next)::value;
        constexpr bool kNext = decltype(next)::value;
        if constexpr (kNext) {
            if (p + kStages - 1 <= np)
                __builtin_amdgcn_s_waitcnt(0x0F70 | ((kStages - 3) * LPT));  // pair p + 2's may stay
            else
                __builtin_amdgcn_s_waitcnt(0x0F70);                          // vmcnt(0)
            asm volatile("s_barrier" ::: "memory");
            if (p + kStages - 1 < np) issue(p + kStages - 1);
        }
        u32x4 k0[NL], k1[NL], va[NG];
        f32x4 N0[kQB], N1[kQB];
        if constexpr (kNext) read_k(p + 1, k0, k1);
        read_v(p, va);
        // A.  Near the diagonal or the sequence end every block is masked; a block that
        // sees no key of the pair adds exact zeros (its maximum is already finite:
        // every column sees key 0 in pair 0).
        // Masked pairs skip the blocks that see no key of the pair (past a block's last
        // row, or an empty block): a fully masked pair would only add exact zeros.
        const uint32_t act = kEdge ? active_at(p) : ~0u;
        const uint32_t act_next = kEdgeNext ? active_at(p + 1) : ~0u;
        bf16x8 pB[kQB];
        pair_weights<D, kQB, kEdge>(pB, st, x, cs, act);
        if constexpr (kNext) {
            // 2 NG V reads were issued after the K reads: at most min(2 NG, 15) LDS reads
            // outstanding leaves every K read done
#pragma unroll
            for (int k = 0; k < NL; ++k)
                asm volatile("s_waitcnt lgkmcnt(%2)" : "+v"(k0[k]), "+v"(k1[k]) : "i"(2 * NG > 15 ? 15 : 2 * NG));
            pair_scores<D, kQB, kEdgeNext>(N0, N1, q, k0, k1, act_next);
            interleave_mfma_valu<4 * NL * kQB, 3>();
        }
        // B
        pair_pv<D, kQB, kEdge, kEdge>(st, pB, va, p * kPairKeys, L, j, act);
        if constexpr (kNext) {
            float mx[kQB];
            const bool any = pair_max<D, kQB, kEdgeNext, kEdgeNext>(st, x, mx, N0, N1,
                                                                    (p + 1) * kPairKeys, lim, cs,
                                                                    j, act_next);
            interleave_mfma_valu<(NG + 1) * kQB, 2>();
            if (__ballot(any)) rescale<D, kQB>(st, mx);
        }
    };
    int p = 0;
    for (; p + 1 < pf; ++p) pair_step(p, std::false_type{}, std::false_type{}, std::true_type{});
    if (p < pf) {
        pair_step(p, std::false_type{}, std::true_type{}, std::true_type{});
        ++p;
    }
    for (; p < np - 1; ++p) pair_step(p, std::true_type{}, std::true_type{}, std::true_type{});
    pair_step(np - 1, std::true_type{}, std::true_type{}, std::false_type{});

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

template <int D, bool Half>
hipError_t launch_group_size(int group, PrefillArgs& a, hipStream_t st) {
    const dim3 block(kThreads);
    const int nsh = a.num_seqs * a.num_kv_heads;
    const dim3 grid(kXcds * ((nsh + kXcds - 1) / kXcds) * a.qgroups);
    switch (group) {
        case 1: hipLaunchKernelGGL((prefill_kernel<D, 1, Half>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((prefill_kernel<D, 2, Half>), grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((prefill_kernel<D, 4, Half>), grid, block, 0, st, a); break;
        case 8: hipLaunchKernelGGL((prefill_kernel<D, 8, Half>), grid, block, 0, st, a); break;
        case 16: hipLaunchKernelGGL((prefill_kernel<D, 16, Half>), grid, block, 0, st, a); break;
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
    const bool half = a.block_size == 8;
    if (head_dim == 128)
        return half ? launch_group_size<128, true>(group, a, stream)
                    : launch_group_size<128, false>(group, a, stream);
    if (head_dim == 64)
        return half ? launch_group_size<64, true>(group, a, stream)
                    : launch_group_size<64, false>(group, a, stream);
    return hipErrorInvalidValue;
}

}  // namespace pkv
