// Paged decode attention for gfx950: pass 1 (block-table gather, QK^T, online
// softmax, PV) and the log-sum-exp merge of split sequences, either inside pass 1
// (the default, one kernel) or as a separate pass 2.
//
// The kernels and their launchers; decode_variant.hip instantiates them, one
// (load policy, decode step, block size 8) variant per object so the variants
// compile in parallel, and kernels_decode.hip picks the variant for a call.
//
// What is computed: one new query token per sequence attends over every cached
// token of its sequence (ksqn.cn "大模型推理性能优化：PagedAttention与Continuous
// Batching原理与实践", section 2), whose keys/values sit in fixed-size blocks
// scattered through one pool and are found through the sequence's block table
// (same page, section 2.2; hihuo.com "vLLM 原理：PagedAttention 和 Continuous
// Batching", PagedAttention > 工作原理 > 1. 页表管理).  Batches are ragged (ksqn.cn
// page, section 2.3, item 3).
//
// Work split ("units"): per work row (a KV head for the group kernel, a query
// head for the per-head kernel) the sequences' 16-token tiles are laid end to
// end.  With at least one unit per row, every row is cut into the same
// num_units / rows ranges (the aligned split), so the units of one range cover
// the same tiles in every row.  The ranges are equal in cost, where a sequence
// costs its tiles plus one tile for opening and closing its piece; with fewer
// units than rows, the rows are laid one after another and the whole line is
// cut into num_units ranges of equal tile count.  One wavefront owns one range:
// even work whatever the length mix.
// Under the aligned split, the rows of one range (up to eight) run as the waves
// of one workgroup and meet once per tile, so the adjacent 4 KiB head slices of
// a block are requested together.  A sequence that a range holds whole is
// finished in place; a sequence cut by range ends leaves partial (max, sum,
// accumulator) records.  In the single-kernel form each holder then adds one to
// an arrival count kept for the sequence's last holder; the holder whose add
// completes it merges the records with the log-sum-exp rule and resets the
// count.  In the two-kernel form pass 2 does the same merge, in the same order.
// Every wave scans the context lengths itself to find its range, so no
// planning kernel runs first.
//
// Two pass-1 kernels:
//  * per-head (VALU): one query head per row.  A lane owns one token of the
//    tile for K (dot product over 32 dims, finished with two cross-row adds)
//    and four tokens of two dims for V (fp32 FMA); used for G == 1 and for
//    every fp32 case.
//  * group (MFMA): one KV head per row with its G query heads.  S = K Q^T is
//    a 16x16x32 bf16 MFMA per 32 dims (Q columns repeat with period G), and
//    O^T = V^T P^T a 16x16x16 bf16 MFMA per 16 dims; accumulation in fp32.
//
// Scores are kept in base-2 units (scale * log2 e folded into one multiply)
// so that exp2 maps to v_exp_f32.

#pragma once

#include "kernels_common.h"
#include "pagedkv_internal.h"

namespace pkv {
namespace {

// Partial records are written and read at device scope (write-through past this
// XCD's L2, reads from the device-coherent level), so a record written by one
// XCD can be merged by another in the same launch without cache maintenance.
//
// The in-launch merge hands records between workgroups with relaxed device-scope
// atomics only: a holder's record stores, then `s_waitcnt vmcnt(0)`, then a relaxed
// fetch-add on the arrival count; the merger reads the records with relaxed
// device-scope loads after it has seen the count complete.  The language memory
// model orders none of this (there is no release on the add and no acquire before
// the reads).  It is correct on gfx950 because (1) device-scope atomic stores are
// written through to the device-coherent level, (2) on gfx9 the vector-memory
// counter also counts stores, and waiting it to zero waits for their completion
// acknowledgement, and (3) device-scope atomic loads are not served from a
// non-coherent cache.  Agent-scope release/acquire fences would add an L2
// write-back and invalidate per piece.  The assumption is tied to this ISA, so
// the file refuses to compile for any other target.
#if defined(__HIP_DEVICE_COMPILE__) && !defined(__gfx950__)
#error "the decode kernels' in-launch merge relies on gfx950 memory behaviour; build for gfx950 only"
#endif
// Word 3 of a raw buffer resource on gfx9-family targets: 32-bit data format, no
// swizzle (the hardware's documented value for untyped buffer loads).
constexpr int kBufferRsrcWord3 = 0x00020000;

__device__ __forceinline__ void store_dev(float* p, float v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void store_dev2(float* p, float lo, float hi) {
    const uint64_t w = static_cast<uint64_t>(__float_as_uint(lo)) |
                       (static_cast<uint64_t>(__float_as_uint(hi)) << 32);
    __hip_atomic_store(reinterpret_cast<uint64_t*>(p), w, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float load_dev(const float* p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------------
// One 16-token tile folded into a group accumulator with the matrix cores.
//
// Sixteen columns share the K/V tile of one KV head: the G query heads of that
// head, repeated with period G.  Lane l = 16 j + i owns column i.
//   S^T = K Q^T: v_mfma_f32_16x16x32_bf16, one per 32 dims; A = the K tile as
//     loaded (token i, dims 32 s + 8 j ..), B = the column's query (same dims).
//     Lane (j, i) gets the scores of tokens 4 j .. 4 j + 3 for column i.
//   Online softmax per column in base 2 (scores times scale * log2 e); P is
//     rounded to bf16 in the accumulator layout, which is the B operand of
//   O^T = V^T P^T: v_mfma_f32_16x16x16_bf16, one per 16 dims, fp32 accumulate.
//     acc[g][r] is dim 16 g + 4 j + r of column i.
// Token k of tile t is visible when 16 t + k < lim.  Value rows of tokens at or past
// vlim (the sequence length) are zeroed first: their slots may hold anything, and
// a zero weight times a NaN would still poison the sum; vlim must be uniform over
// the wave.  Every column must see at least one token of the first tile it folds, so
// that its running max is finite.
template <int D>
struct GroupAcc {
    float m, l;
    f32x4 acc[D / 16];
};

template <int D>
__device__ __forceinline__ void group_tile(GroupAcc<D>& st, const u32x4 (&q)[D / 32],
                                           const u32x4* kb, const u32x4* vb, int t, int lim,
                                           int vlim, float scale_log2e, int lane) {
    constexpr int NL = D / 32, NG = D / 16;
    const int j = lane >> 4;
    f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
    for (int s = 0; s < NL; ++s)
        S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[s]),
                                                    __builtin_bit_cast(bf16x8, q[s]), S, 0, 0, 0);
    const int tok0 = t * kTile + 4 * j;
    float sc[4];
#pragma unroll
    for (int r = 0; r < 4; ++r) sc[r] = (tok0 + r < lim) ? S[r] * scale_log2e : kNegInf;
    float tmax = fmaxf(fmaxf(sc[0], sc[1]), fmaxf(sc[2], sc[3]));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 16));
    tmax = fmaxf(tmax, __shfl_xor(tmax, 32));
    const float m_new = fmaxf(st.m, tmax);
    const float alpha = fast_exp2(st.m - m_new);
    uint32_t pb[4];
    float psum = 0.f;
#pragma unroll
    for (int r = 0; r < 4; ++r) {
        pb[r] = bf16_rne_finite(fast_exp2(sc[r] - m_new));
        psum += __uint_as_float(pb[r] << 16);
    }
    st.l = st.l * alpha + psum;
    st.m = m_new;
    const s16x4 pB = __builtin_bit_cast(
        s16x4, (unsigned __attribute__((ext_vector_type(2)))){pb[0] | (pb[1] << 16),
                                                              pb[2] | (pb[3] << 16)});
#pragma unroll
    for (int g = 0; g < NG; ++g) st.acc[g] *= alpha;
    const bool last = t * kTile + kTile > vlim;
    uint32_t mask01 = 0xffffffffu, mask23 = 0xffffffffu;
    if (last) {
        const int nv = vlim - tok0;
        mask01 = (nv > 0 ? 0x0000ffffu : 0u) | (nv > 1 ? 0xffff0000u : 0u);
        mask23 = (nv > 2 ? 0x0000ffffu : 0u) | (nv > 3 ? 0xffff0000u : 0u);
    }
#pragma unroll
    for (int mm = 0; mm < NL; ++mm) {
#pragma unroll
        for (int e = 0; e < 2; ++e) {
            const unsigned w0 = vb[mm][2 * e] & mask01;
            const unsigned w1 = vb[mm][2 * e + 1] & mask23;
            const s16x4 vA = __builtin_bit_cast(
                s16x4, (unsigned __attribute__((ext_vector_type(2)))){w0, w1});
            st.acc[2 * mm + e] =
                __builtin_amdgcn_mfma_f32_16x16x16bf16_1k(vA, pB, st.acc[2 * mm + e], 0, 0, 0);
        }
    }
}

// Context length of sequence i, clamped to what its table row can address.
__device__ __forceinline__ int ctx_of(const DecodeArgs& a, int i) {
    const int cap = a.max_blocks * a.block_size;
    return min(max(a.context_lens[i], 0), cap);
}

__device__ __forceinline__ int tiles_of(int ctx) { return (ctx + kTile - 1) / kTile; }

// Lane k of the window holds table entry e_lo + k (entries past e_last read as 0).
// IDs outside [0, N) become 0 so that a bad table never addresses outside the pool.
__device__ __forceinline__ int load_window(const int32_t* bt, int e_lo, int e_last, int lane,
                                           int num_blocks) {
    const int e = e_lo + lane;
    int b = e <= e_last ? bt[e] : 0;
    return (static_cast<unsigned>(b) < static_cast<unsigned>(num_blocks)) ? b : 0;
}

// Zero every query head of sequence `seq` (a sequence with no cached tokens).
template <typename T, int D>
__device__ void write_zero_seq(const DecodeArgs& a, int seq, int lane) {
    T* o = static_cast<T*>(a.out) + static_cast<size_t>(seq) * a.num_q_heads * D;
    for (int k = lane; k < a.num_q_heads * D; k += kWave) o[k] = 0;
}

// ---------------------------------------------------------------------------------
// A path supplies, for one work row (its query heads, its KV head):
//   Q, Acc              query registers and running softmax state
//   kv_head(a, row)     the KV head a row reads
//   load_q / reset      start a piece
//   tile                fold one 16-token tile into Acc
//   finish              write the piece: `out` when the unit holds the whole
//                       sequence, else a partial (acc, max, sum) record
//
// Per-head path (VALU).  Lane l = 16 j + i.
//   K load s: token i, dims (4s + j) X + x       (x < X)
//   V load m: tokens 4j .. 4j+3, dims 16E m + 16e + i   (e < E)
template <typename T, int D>
struct HeadPath {
    static constexpr int X = 16 / sizeof(T);
    static constexpr int E = X / 4;
    static constexpr int NL = D * static_cast<int>(sizeof(T)) / 64;  // 16-B loads per lane per tile
    static constexpr int TILE_U4 = D * static_cast<int>(sizeof(T));   // tile size in 16-B units
    static constexpr bool kBf16 = sizeof(T) == 2;
    static constexpr int GH = 1;  // query heads per row

    struct Q {
        u32x4 v[NL];
    };
    struct Acc {
        float m, l;
        float acc[NL][E];
    };

    static __device__ __forceinline__ int kv_head(const DecodeArgs& a, int row) {
        return row / a.group;
    }

    static __device__ __forceinline__ void load_q(const DecodeArgs& a, Q& q, int row, int seq,
                                                  int lane) {
        const int j = lane >> 4;
        const T* qrow = static_cast<const T*>(a.q) + (static_cast<size_t>(seq) * a.num_q_heads + row) * D;
#pragma unroll
        for (int s = 0; s < NL; ++s) q.v[s] = *reinterpret_cast<const u32x4*>(qrow + (4 * s + j) * X);
    }

    static __device__ __forceinline__ void reset(Acc& st) {
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int mm = 0; mm < NL; ++mm)
#pragma unroll
            for (int e = 0; e < E; ++e) st.acc[mm][e] = 0.f;
    }

    static __device__ __forceinline__ void tile(const DecodeArgs& a, Acc& st, const Q& q,
                                                const u32x4* kb, const u32x4* vb, int t, int ctx,
                                                int lane) {
        const int j = lane >> 4, i = lane & 15;
        // QK: partial dot over this lane's dims, then across the four rows.
        float part = 0.f;
#pragma unroll
        for (int s = 0; s < NL; ++s) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if constexpr (kBf16) {
                    part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kb[s][w]),
                                                           as_bf16x2(q.v[s][w]), part, false);
                } else {
                    part = __builtin_fmaf(__uint_as_float(kb[s][w]), __uint_as_float(q.v[s][w]),
                                          part);
                }
            }
        }
        part += __shfl_xor(part, 16);
        part += __shfl_xor(part, 32);
        const int tok0 = t * kTile;
        const float sc = (tok0 + i < ctx) ? part * a.scale_log2e : kNegInf;
        float tmax = sc;
        tmax = fmaxf(tmax, __shfl_xor(tmax, 1));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 2));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 4));
        tmax = fmaxf(tmax, __shfl_xor(tmax, 8));
        const float m_new = fmaxf(st.m, tmax);
        const float alpha = fast_exp2(st.m - m_new);
        const float p = fast_exp2(sc - m_new);
        st.l = st.l * alpha + p;
        st.m = m_new;
        // Weights of tokens 4j + r, taken from the lanes of this row that own them.
        float p4[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) p4[r] = __shfl(p, (j << 4) + 4 * j + r);
        const bool last = tok0 + kTile > ctx;
        const int nvalid = ctx - (tok0 + 4 * j);  // tokens of this lane's quad inside ctx
#pragma unroll
        for (int mm = 0; mm < NL; ++mm) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float v[4];
                if constexpr (kBf16) {
                    v[0] = bf_lo(vb[mm][2 * e]);
                    v[1] = bf_hi(vb[mm][2 * e]);
                    v[2] = bf_lo(vb[mm][2 * e + 1]);
                    v[3] = bf_hi(vb[mm][2 * e + 1]);
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = __uint_as_float(vb[mm][r]);
                }
                if (last) {
#pragma unroll
                    for (int r = 0; r < 4; ++r) v[r] = r < nvalid ? v[r] : 0.f;
                }
                float acc = st.acc[mm][e] * alpha;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc = __builtin_fmaf(p4[r], v[r], acc);
                st.acc[mm][e] = acc;
            }
        }
    }

    static __device__ __forceinline__ void finish(const DecodeArgs& a, Acc& st, int row, int seq,
                                                  bool whole, float* rec, int lane) {
        const int j = lane >> 4, i = lane & 15;
        float L = st.l;
        L += __shfl_xor(L, 1);
        L += __shfl_xor(L, 2);
        L += __shfl_xor(L, 4);
        L += __shfl_xor(L, 8);
#pragma unroll
        for (int mm = 0; mm < NL; ++mm) {
#pragma unroll
            for (int e = 0; e < E; ++e) {
                float v = st.acc[mm][e];
                v += __shfl_xor(v, 16);
                v += __shfl_xor(v, 32);
                st.acc[mm][e] = v;
            }
        }
        if (j != 0) return;
        if (whole) {
            T* o = static_cast<T*>(a.out) + (static_cast<size_t>(seq) * a.num_q_heads + row) * D;
            const float inv = 1.f / L;
#pragma unroll
            for (int mm = 0; mm < NL; ++mm)
#pragma unroll
                for (int e = 0; e < E; ++e) store_out<T>(o + 16 * E * mm + 16 * e + i, st.acc[mm][e] * inv);
        } else {
#pragma unroll
            for (int mm = 0; mm < NL; ++mm)
#pragma unroll
                for (int e = 0; e < E; ++e) store_dev(rec + 16 * E * mm + 16 * e + i, st.acc[mm][e]);
            if (i == 0) {
                store_dev(rec + D, st.m);
                store_dev(rec + D + 1, L);
            }
        }
    }
};

// ---------------------------------------------------------------------------------
// Group path (MFMA, bf16).  Lane l = 16 j + i; query column i holds head i % G.
//   K load s: token i, dims 32 s + 8 j + x  -> A operand of S = K Q^T (16x16x32)
//   S[r]    : token 4 j + r, head column i  -> B operand of O^T = V^T P^T (16x16x16)
//   V load m: tokens 4j .. 4j+3 of dims 32 m + i (words 0,1) and 32 m + 16 + i (words 2,3)
//             -> A operands of the two 16-dim groups 2m, 2m+1
//   acc[g][r]: dim 16 g + 4 j + r, head column i
template <int D, int G>
struct GroupPath {
    using T = uint16_t;
    static constexpr int GH = G;  // query heads per row
    static constexpr int NL = D / 32;  // 16-B loads per lane per tile (K and V)
    static constexpr int NG = D / 16;  // 16-dim output groups
    static constexpr int TILE_U4 = D * 2;

    struct Q {
        u32x4 v[NL];
    };
    using Acc = GroupAcc<D>;

    static __device__ __forceinline__ int kv_head(const DecodeArgs&, int row) { return row; }

    static __device__ __forceinline__ void load_q(const DecodeArgs& a, Q& q, int row, int seq,
                                                  int lane) {
        const int j = lane >> 4, i = lane & 15;
        const T* qrow = static_cast<const T*>(a.q) +
                        (static_cast<size_t>(seq) * a.num_q_heads + row * G + (i % G)) * D;
#pragma unroll
        for (int s = 0; s < NL; ++s) q.v[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * j);
    }

    static __device__ __forceinline__ void reset(Acc& st) {
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) st.acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
    }

    static __device__ __forceinline__ void tile(const DecodeArgs& a, Acc& st, const Q& q,
                                                const u32x4* kb, const u32x4* vb, int t, int ctx,
                                                int lane) {
        group_tile<D>(st, q.v, kb, vb, t, ctx, ctx, a.scale_log2e, lane);
    }

    static __device__ __forceinline__ void finish(const DecodeArgs& a, Acc& st, int row, int seq,
                                                  bool whole, float* rec, int lane) {
        const int j = lane >> 4, i = lane & 15;
        float L = st.l;
        L += __shfl_xor(L, 16);
        L += __shfl_xor(L, 32);
        if (i >= G) return;
        if (whole) {
            T* o = static_cast<T*>(a.out) + (static_cast<size_t>(seq) * a.num_q_heads + row * G + i) * D;
            const float inv = 1.f / L;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const uint32_t lo = bf16_rne(st.acc[g][0] * inv) | (uint32_t(bf16_rne(st.acc[g][1] * inv)) << 16);
                const uint32_t hi = bf16_rne(st.acc[g][2] * inv) | (uint32_t(bf16_rne(st.acc[g][3] * inv)) << 16);
                *reinterpret_cast<uint2*>(o + 16 * g + 4 * j) = make_uint2(lo, hi);
            }
        } else {
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                store_dev2(rec + i * D + 16 * g + 4 * j, st.acc[g][0], st.acc[g][1]);
                store_dev2(rec + i * D + 16 * g + 4 * j + 2, st.acc[g][2], st.acc[g][3]);
            }
            if (j == 0) {
                store_dev(rec + G * D + i, st.m);
                store_dev(rec + G * D + G + i, L);
            }
        }
    }
};

// ---------------------------------------------------------------------------------
// Log-sum-exp merge of the partial records of one split (sequence, row), pieces
// held by units us .. ue (unit us keeps it in record slot 1, the others in slot 0):
//   M = max_p m_p;  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
// GH heads share a row.  Pair k = (piece us + k / GH, head k % GH).  First each
// lane folds its pairs' (m, l) with a running maximum; GH divides the wave width,
// so lane L only ever sees head L % GH, and an xor reduction over lanes GH apart
// gives every lane its head's M and sum.  Then each lane owns K = GH * D / 64
// output elements; the accumulators of up to four pieces are requested at once,
// and their weights come from the lanes holding the pairs (or from memory when a
// split has more than 64 pairs).
template <typename T, int D, int GH>
__device__ __forceinline__ void merge_pieces(const DecodeArgs& a, int row, int seq, int us, int ue,
                                             int lane) {
    constexpr int K = GH * D / kWave;
    static_assert(K >= 1 && (GH * D) % kWave == 0 && kWave % GH == 0, "merge shape");
    constexpr int kMOff = GH * D;  // record: [GH][D] acc, [GH] m, [GH] l
    constexpr size_t pf = static_cast<size_t>(GH * D + ((2 * GH + 3) & ~3));
    auto piece = [&](int p) -> const float* {
        return a.pieces + (static_cast<size_t>(p) * 2 + (p == us ? 1 : 0)) * pf;
    };
    const int np = ue - us + 1;
    const int pairs = np * GH;
    // Accumulators of NB pieces are requested at once (fewer when a lane holds many
    // elements, to bound the registers); the sum runs in piece order either way.  The
    // first NB are requested together with the (m, l) pairs below.
    constexpr int NB = K >= 32 ? 1 : K >= 16 ? 2 : 4;
    const int nb0 = min(NB, np);
    float v0[NB][K];
#pragma unroll
    for (int t = 0; t < NB; ++t) {
        const float* r = piece(us + min(t, nb0 - 1));
#pragma unroll
        for (int c = 0; c < K; ++c) v0[t][c] = t < nb0 ? load_dev(r + lane + kWave * c) : 0.f;
    }
    // (m, l) of this lane's first pair; kept for the weights below
    float m0 = kNegInf, l0 = 0.f;
    if (lane < pairs) {
        const float* r = piece(us + lane / GH);
        m0 = load_dev(r + kMOff + lane % GH);
        l0 = load_dev(r + kMOff + GH + lane % GH);
    }
    float M = m0, den = l0;
    for (int k = lane + kWave; k < pairs; k += kWave) {  // splits with more than 64 pairs
        const float* r = piece(us + k / GH);
        const float m = load_dev(r + kMOff + k % GH);
        const float mn = fmaxf(M, m);
        den = den * fast_exp2(M - mn) + fast_exp2(m - mn) * load_dev(r + kMOff + GH + k % GH);
        M = mn;
    }
#pragma unroll
    for (int o = GH; o < kWave; o <<= 1) {
        const float Mo = __shfl_xor(M, o), Do = __shfl_xor(den, o);
        const float mn = fmaxf(M, Mo);
        // a side with no pairs has M = -inf and den = 0: guard its 2^(-inf - -inf)
        den = (M == kNegInf ? 0.f : den * fast_exp2(M - mn)) +
              (Mo == kNegInf ? 0.f : Do * fast_exp2(Mo - mn));
        M = mn;
    }
    // weight of this lane's first pair (pairs < 64: every weight is in some lane)
    const float w0 = fast_exp2(m0 - M);
    float Mh[K], acc[K];
#pragma unroll
    for (int c = 0; c < K; ++c) {
        Mh[c] = __shfl(M, (kWave * c) / D);  // element c of this lane is lane + 64 c, head 64 c / D
        acc[c] = 0.f;
    }
#pragma unroll
    for (int t = 0; t < NB; ++t) {
        if (t >= nb0) break;
        const int pk = t * GH;
#pragma unroll
        for (int c = 0; c < K; ++c) {
            const int h = (kWave * c) / D;
            const float w = pairs <= kWave ? __shfl(w0, pk + h)
                                           : fast_exp2(load_dev(piece(us + t) + kMOff + h) - Mh[c]);
            acc[c] = __builtin_fmaf(w, v0[t][c], acc[c]);
        }
    }
    int p = us + nb0;
    for (; p + NB <= ue + 1; p += NB) {
        float v[NB][K];
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const float* r = piece(p + t);
#pragma unroll
            for (int c = 0; c < K; ++c) v[t][c] = load_dev(r + lane + kWave * c);
        }
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int pk = (p + t - us) * GH;
#pragma unroll
            for (int c = 0; c < K; ++c) {
                const int h = (kWave * c) / D;
                const float w = pairs <= kWave ? __shfl(w0, pk + h)
                                               : fast_exp2(load_dev(piece(p + t) + kMOff + h) - Mh[c]);
                acc[c] = __builtin_fmaf(w, v[t][c], acc[c]);
            }
        }
    }
    for (; p <= ue; ++p) {
        const float* r = piece(p);
        float v[K];
#pragma unroll
        for (int c = 0; c < K; ++c) v[c] = load_dev(r + lane + kWave * c);
        const int pk = (p - us) * GH;
#pragma unroll
        for (int c = 0; c < K; ++c) {
            const int h = (kWave * c) / D;
            const float w = pairs <= kWave ? __shfl(w0, pk + h) : fast_exp2(load_dev(r + kMOff + h) - Mh[c]);
            acc[c] = __builtin_fmaf(w, v[c], acc[c]);
        }
    }
    const int qh0 = row * GH;  // group rows hold heads row*G..; per-head rows hold head `row`
    T* o = static_cast<T*>(a.out) + (static_cast<size_t>(seq) * a.num_q_heads + qh0) * D;
#pragma unroll
    for (int c = 0; c < K; ++c) store_out<T>(o + lane + kWave * c, acc[c] / __shfl(den, (kWave * c) / D));
}

// ---------------------------------------------------------------------------------
// A decode step's new token inside a tile, for the lanes that hold its place.  Both
// paths read a tile in one register layout (it follows from the cache layout): lane
// l = 16 j + i holds, for K load s, token i at dims (4 s + j) X .. (4 s + j) X + X - 1,
// and for V load m, tokens 4 j .. 4 j + 3 at dims 16 E m + 16 e + i (e < E), each
// 16-byte group holding for each e the four tokens' values (element e * 4 + token % 4).
// So for the token at position p of the tile, the lanes with i == p load its K groups
// from the new row instead of the cache (the tile's own bytes there are not needed),
// and the lanes with j == p / 4 load one value per (m, e) of its V row, merged into
// the groups once the tile has arrived.
template <typename T, int NL>
struct TokenV {
    static constexpr int X = 16 / static_cast<int>(sizeof(T));
    static constexpr int E = X / 4;
    uint32_t v[NL][E];
};

// Every lane issues the same loads on every tile (lanes and tiles without the token
// read a harmless element instead): the number of loads in flight then never
// depends on the tile, so the compiler's waits for a tile never wait for the next
// tile's loads as well.
template <typename T, int NL>
__device__ __forceinline__ void load_token_v(TokenV<T, NL>& tv, const T* vn, const T* dummy, int p,
                                             int lane) {
    constexpr int E = TokenV<T, NL>::E;
    const int j = lane >> 4, i = lane & 15;
    const bool mine = p >= 0 && j == (p >> 2);
    const T* base = mine ? vn + i : dummy;
    const int stride = mine ? 16 : 0;
#pragma unroll
    for (int m = 0; m < NL; ++m)
#pragma unroll
        for (int e = 0; e < E; ++e) tv.v[m][e] = static_cast<uint32_t>(base[stride * (E * m + e)]);
}

template <typename T, int NL>
__device__ __forceinline__ void patch_token_v(u32x4* vb, const TokenV<T, NL>& tv, int p, int lane) {
    const int j = lane >> 4;
    if (j != (p >> 2)) return;
    const int r = p & 3;
#pragma unroll
    for (int m = 0; m < NL; ++m) {
        u32x4 g = vb[m];
        if constexpr (sizeof(T) == 2) {
            // word 2 e + (r >> 1) holds tokens 4 j + 2 (r >> 1) .. + 1 of the e-th dim
            const bool odd = (r >> 1) != 0, high = (r & 1) != 0;
            uint32_t w0 = odd ? g[1] : g[0];
            uint32_t w2 = odd ? g[3] : g[2];
            w0 = high ? ((w0 & 0xffffu) | (tv.v[m][0] << 16)) : ((w0 & 0xffff0000u) | tv.v[m][0]);
            w2 = high ? ((w2 & 0xffffu) | (tv.v[m][1] << 16)) : ((w2 & 0xffff0000u) | tv.v[m][1]);
            if (odd) {
                g[1] = w0;
                g[3] = w2;
            } else {
                g[0] = w0;
                g[2] = w2;
            }
        } else {
            // one token per word
            g[0] = r == 0 ? tv.v[m][0] : g[0];
            g[1] = r == 1 ? tv.v[m][0] : g[1];
            g[2] = r == 2 ? tv.v[m][0] : g[2];
            g[3] = r == 3 ? tv.v[m][0] : g[3];
        }
        vb[m] = g;
    }
}

// ---------------------------------------------------------------------------------
// Walking a unit's tiles.  The line of tiles is addressed by a cursor (row,
// sequence, tile inside the sequence).  A chunk describes up to 64 consecutive
// tiles of the walk, one per lane, with everything the loop needs to fetch and
// fold that tile: its sequence, row, tile index, the sequence's context length
// and the tile's position in the cache (block-table entry already applied).
// Building a chunk reads the context lengths of the next 64 sequences and the
// table entries of its tiles in one parallel round each, so the tile loop
// itself never waits on a dependent table read, also across sequence ends.
struct Cursor {
    int row, seq, t0;
};

struct Chunk {
    int n;       // tiles held (uniform)
    int seq;     // lane k: sequence of tile k
    int tile;    // lane k: tile index inside its sequence
    int row;     // lane k: work row
    int ctx;     // lane k: context length of its sequence
    int toff;    // lane k: tile index in the cache, (block * tpb + tile % tpb) * Hkv + kv head;
                 // 8-token blocks: the 8-token tile of the tile's first block, block * Hkv + kv head
    int toff2;   // lane k (8-token blocks): the same for the tile's second block
    int wtoff;   // lane k (decode step): tile index the tile is written to, -1 = none
    int ptok;    // lane k (decode step): position of the new token in the tile, -1 = none
    Cursor next; // where the walk continues after the chunk (uniform)
};

// Uniform copy of one lane of a chunk.
struct TileRef {
    int seq, tile, row, ctx, toff, toff2, wtoff, ptok;
};

template <bool Step, bool Half>
__device__ __forceinline__ TileRef tile_ref(const Chunk& c, int k) {
    TileRef r;
    r.seq = __builtin_amdgcn_readlane(c.seq, k);
    r.tile = __builtin_amdgcn_readlane(c.tile, k);
    r.row = __builtin_amdgcn_readlane(c.row, k);
    r.ctx = __builtin_amdgcn_readlane(c.ctx, k);
    r.toff = __builtin_amdgcn_readlane(c.toff, k);
    r.toff2 = Half ? __builtin_amdgcn_readlane(c.toff2, k) : r.toff;
    if constexpr (Step) {
        r.wtoff = __builtin_amdgcn_readlane(c.wtoff, k);
        r.ptok = __builtin_amdgcn_readlane(c.ptok, k);
    } else {
        r.wtoff = -1;
        r.ptok = -1;
    }
    return r;
}

// The chunk of at most min(64, remaining) tiles starting at cursor c.  Rows wrap
// after sequence S - 1; sequences with no tiles are passed over.  Block IDs
// outside [0, N) are replaced by 0 so a bad table never addresses outside the pool.
// Half: blocks of 8 tokens, so 16-token tile t of a sequence is blocks 2t and 2t + 1
// of its table; when the sequence ends inside block 2t, the second half reads block
// 2t again (its tokens are past the context and never weighted), so no table entry
// past the sequence's last block is read.
template <class Path, bool Step, bool Half>
__device__ __forceinline__ Chunk build_chunk(const DecodeArgs& a, Cursor c, int remaining,
                                             int lane) {
    const int S = a.num_seqs;
    // lane k looks at the k-th sequence from the cursor
    int sk = c.seq + lane;
    const int rk = c.row + sk / S;
    sk %= S;
    const int ctx_k = rk < a.rows ? ctx_of(a, sk) : 0;
    int n = tiles_of(ctx_k);
    if (lane == 0) n -= c.t0;
    const int incl = wave_inclusive_scan(n, lane);
    const int excl = incl - n;
    const int avail = __builtin_amdgcn_readlane(incl, kWave - 1);
    Chunk ch;
    ch.n = min(min(kWave, remaining), avail);
    // tile k belongs to the source lane j with excl_j <= k < incl_j
    int j = 0;
    for (int src = 0; src < kWave; ++src) {
        const int lo = __builtin_amdgcn_readlane(excl, src);
        if (lo >= ch.n) break;
        if (lane >= lo && lane < __builtin_amdgcn_readlane(incl, src)) j = src;
    }
    const int tin = lane - __shfl(excl, j) + (j == 0 ? c.t0 : 0);
    const int ssk = __shfl(sk, j);
    const int rr = __shfl(rk, j);
    ch.seq = ssk;
    ch.row = rr;
    ch.tile = tin;
    ch.ctx = __shfl(ctx_k, j);
    int toff = 0, toff2 = 0, wtoff = -1, ptok = -1;
    if (Half && lane < ch.n) {
        const int32_t* bt = a.block_tables + static_cast<size_t>(ssk) * a.max_blocks;
        const int c = ch.ctx;
        const int e0 = 2 * tin;
        const int e1 = min(e0 + 1, (c - 1) >> 3);  // the sequence's last block at most
        int blk0 = bt[e0];
        int blk1 = e1 > e0 ? bt[e1] : blk0;
        int wblk = -1;
        if constexpr (Step) {
            // The sequence's last block (entry (c - 1) / 8) lies in the new token's tile:
            // it is read from the step's read block and, under copy-on-write, written
            // whole to the write block; in place only the token was new (scattered at
            // the start).
            if (c > 0 && tin == (c - 1) >> 4) {
                const u32x4 info = *reinterpret_cast<const u32x4*>(a.seq_info + 4 * ssk);
                if (static_cast<int>(info[2]) & 1) {
                    const int last = (c - 1) >> 3;
                    if (last == e0) blk0 = static_cast<int>(info[0]);
                    if (last == e1) blk1 = static_cast<int>(info[0]);
                    wblk = static_cast<int>(info[1]);
                    ptok = (c - 1) & (kTile - 1);
                }
            }
        }
        blk0 = static_cast<unsigned>(blk0) < static_cast<unsigned>(a.num_blocks) ? blk0 : 0;
        blk1 = static_cast<unsigned>(blk1) < static_cast<unsigned>(a.num_blocks) ? blk1 : 0;
        const int kvh = Path::kv_head(a, rr);
        toff = blk0 * a.num_kv_heads + kvh;
        toff2 = blk1 * a.num_kv_heads + kvh;
        if (static_cast<unsigned>(wblk) < static_cast<unsigned>(a.num_blocks))
            wtoff = wblk * a.num_kv_heads + kvh;
        else
            ptok = -1;
    }
    if (!Half && lane < ch.n) {
        const int tpb = a.tiles_per_block;
        const int e = tin / tpb;
        int blk = a.block_tables[static_cast<size_t>(ssk) * a.max_blocks + e];
        int wblk = -1;
        if constexpr (Step) {
            // A tile of the last block of a sequence with a new token: that block (and,
            // under copy-on-write, the source it is read from) comes from the step's
            // metadata, not the table.  In place, only the new token's tile is written
            // back; under copy-on-write every tile of the block goes to the copy.
            const int c = ch.ctx;
            if (c > 0 && e == (c - 1) / (tpb * kTile)) {
                const u32x4 info = *reinterpret_cast<const u32x4*>(a.seq_info + 4 * ssk);
                const int flags = static_cast<int>(info[2]);
                if (flags & 1) {
                    const bool tok_tile = tin == (c - 1) / kTile;
                    blk = static_cast<int>(info[0]);
                    if ((flags & 2) || tok_tile) wblk = static_cast<int>(info[1]);
                    if (tok_tile) ptok = (c - 1) & (kTile - 1);
                }
            }
        }
        blk = static_cast<unsigned>(blk) < static_cast<unsigned>(a.num_blocks) ? blk : 0;
        const int kvh = Path::kv_head(a, rr);
        toff = (blk * tpb + (tin - e * tpb)) * a.num_kv_heads + kvh;
        if (static_cast<unsigned>(wblk) < static_cast<unsigned>(a.num_blocks))
            wtoff = (wblk * tpb + (tin - e * tpb)) * a.num_kv_heads + kvh;
        else
            ptok = -1;
    }
    ch.toff = toff;
    ch.toff2 = toff2;
    ch.wtoff = wtoff;
    ch.ptok = ptok;
    // the walk after the chunk
    if (ch.n < avail) {
        const unsigned long long past = __ballot(incl > ch.n);
        const int jn = __ffsll(static_cast<long long>(past)) - 1;
        ch.next.seq = __builtin_amdgcn_readlane(sk, jn);
        ch.next.row = __builtin_amdgcn_readlane(rk, jn);
        ch.next.t0 = ch.n - __builtin_amdgcn_readlane(excl, jn) + (jn == 0 ? c.t0 : 0);
    } else {
        const int s64 = c.seq + kWave;
        ch.next.row = c.row + s64 / S;
        ch.next.seq = s64 % S;
        ch.next.t0 = 0;
    }
    return ch;
}

// ---------------------------------------------------------------------------------
// Pass 1: one wavefront per unit, NW units (rows of one range) per workgroup.
// The loop keeps the next tile's K/V loads (and, when that tile opens a new
// piece, the new query) in flight while the current tile is folded in.
// Stream: K/V tiles read with non-temporal loads (a template parameter, not a
// runtime branch: the compiler would merge two loads of one address and drop the
// hint).  Half: blocks of 8 tokens (a 16-token tile is read from two blocks).
template <class Path, typename T, int D, int NW, bool Stream, bool Step, bool Half>
__global__ __launch_bounds__(64 * NW) void decode_pass1(DecodeArgs a) {
    constexpr int NL = Path::NL;
    const int lane = threadIdx.x & (kWave - 1);
    if constexpr (Step) {
        // The step's metadata, written by workgroup 0: every sequence's context length,
        // the table entry of its new token's block, and the blocks its last block's
        // tiles are read from and written to.  The flag is released after those
        // writes and every workgroup acquires it before reading any of them.
        // Workgroups are dispatched in index order, so workgroup 0 is resident before
        // any workgroup that waits for it.  The wait is bounded all the same: one that
        // runs past its limit is counted in sync[2] and the workgroup goes on (its
        // results are then unspecified, but every access stays in bounds).  The last
        // workgroup past the flag resets it for the next call.
        if (blockIdx.x == 0) {
            const int B = a.block_size;
            const int cap = a.max_blocks * B;
            for (int i = static_cast<int>(threadIdx.x); i < a.num_seqs; i += 64 * NW) {
                // requested together: these may live in host memory
                const int len_in = a.lens_in[i];
                const int64_t slot = a.new_slots[i];
                const int cs = a.cow_in ? a.cow_in[2 * i] : -1;
                const int cd = a.cow_in ? a.cow_in[2 * i + 1] : -1;
                const int len = min(max(len_in, 0), cap);
                int rb = 0, wb = 0, flags = 0;
                if (len > 0 && slot >= 0 && slot < static_cast<int64_t>(a.num_blocks) * B &&
                    static_cast<int>(slot % B) == (len - 1) % B) {
                    const int blk = static_cast<int>(slot / B);
                    const bool cow = cs >= 0 && cs < a.num_blocks && cd == blk && cs != cd;
                    rb = cow ? cs : blk;
                    wb = blk;
                    flags = 1 | (cow ? 2 : 0);
                    a.tables_dev[static_cast<size_t>(i) * a.max_blocks + (len - 1) / B] = blk;
                }
                a.lens_dev[i] = len_in;
                *reinterpret_cast<u32x4*>(a.seq_info + 4 * i) =
                    u32x4{static_cast<unsigned>(rb), static_cast<unsigned>(wb),
                          static_cast<unsigned>(flags), 0u};
            }
            __syncthreads();
            if (threadIdx.x == 0) __hip_atomic_store(a.sync, 1, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_AGENT);
        }
        // While it waits, every workgroup writes its share of the step's new tokens into
        // their slots (the scatter of the two-call form).  Nothing in this launch reads
        // those bytes: the waves that fold a token's tile take the token from k_new /
        // v_new themselves.  Written now, before the K/V streaming starts, the stores
        // do not compete with it.
        {
            constexpr int X = 16 / static_cast<int>(sizeof(T));
            constexpr int E = X / 4;
            const int G = static_cast<int>(gridDim.x);
            const int B = a.block_size;
            const int tt = Half ? 8 : kTile;  // tokens per tile of the cache layout
            const int tpb = Half ? 1 : a.tiles_per_block;
            const int Hkv = a.num_kv_heads;
            const int cap = a.max_blocks * B;
            const int t_lo = static_cast<int>(static_cast<long long>(a.num_seqs) * blockIdx.x / G);
            const int t_hi = static_cast<int>(static_cast<long long>(a.num_seqs) * (blockIdx.x + 1) / G);
            const int work = (t_hi - t_lo) * Hkv * D;
            T* kwr = static_cast<T*>(const_cast<void*>(a.k_cache));
            T* vwr = static_cast<T*>(const_cast<void*>(a.v_cache));
            for (int w = static_cast<int>(threadIdx.x); w < work; w += 64 * NW) {
                const int pair = w / D, d = w - pair * D;
                const int t = t_lo + pair / Hkv, h = pair - (pair / Hkv) * Hkv;
                const int len = min(max(a.lens_in[t], 0), cap);
                const int64_t slot = a.new_slots[t];
                if (len <= 0 || slot < 0 || slot >= static_cast<int64_t>(a.num_blocks) * B ||
                    static_cast<int>(slot % B) != (len - 1) % B)
                    continue;
                const int64_t blk = slot / B;
                const int o = static_cast<int>(slot - blk * B);
                const int ti = o & (tt - 1), j = ti >> 2, r = ti & 3;
                const size_t tile_base =
                    ((static_cast<size_t>(blk) * tpb + o / tt) * Hkv + h) * (static_cast<size_t>(tt) * D);
                const size_t src = (static_cast<size_t>(t) * Hkv + h) * D;
                const int m = d / (16 * E), ee = (d >> 4) % E, i = d & 15;
                vwr[tile_base + ((((m * (tt / 4) + j) * 16 + i) * E + ee) * 4 + r)] =
                    static_cast<const T*>(a.v_new)[src + d];
                if (d % X == 0)
                    *reinterpret_cast<u32x4*>(kwr + tile_base + ((d / X) * tt + ti) * X) =
                        *reinterpret_cast<const u32x4*>(static_cast<const T*>(a.k_new) + src + d);
            }
        }
        if (threadIdx.x == 0) {
            int spins = 0;
            while (__hip_atomic_load(a.sync, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) == 0) {
                __builtin_amdgcn_s_sleep(2);
                if (++spins > kStepSpinLimit) {
                    __hip_atomic_fetch_add(a.sync + 2, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                    break;
                }
            }
            const int past = __hip_atomic_fetch_add(a.sync + 1, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            if (past == static_cast<int>(gridDim.x) - 1) {
                __hip_atomic_store(a.sync + 1, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
                __hip_atomic_store(a.sync, 0, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
            }
        }
        // One agent-scope acquire per workgroup: it invalidates this CU's and this
        // XCD's caches, and the barrier orders the other waves' reads after it.
        if (threadIdx.x < kWave) __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "agent");
        __syncthreads();
    }
    const int S = a.num_seqs;
    const int W = a.num_units;
    const int R = a.rows;
    const int Wr = a.aligned ? W / R : 0;       // units per row (aligned split)
    const int Wrun = a.aligned ? Wr * R : W;    // units that can hold work
    int u = blockIdx.x;
    if constexpr (NW > 1) {
        // NW rows of one range share a workgroup: wave w takes row (b % (R/NW)) NW + w
        const int rg = R / NW;
        const int wv = uni(static_cast<int>(threadIdx.x) >> 6);
        u = ((static_cast<int>(blockIdx.x) % rg) * NW + wv) * Wr + static_cast<int>(blockIdx.x) / rg;
    }
    const size_t pf = static_cast<size_t>((a.heads_per_row * D + ((2 * a.heads_per_row + 3) & ~3)));
    // Sequences with no cached tokens get zeros; unit u covers sequences i == u (mod Wrun).
    if (u < Wrun)
        for (int i = u; i < S; i += Wrun)
            if (ctx_of(a, i) == 0) write_zero_seq<T, D>(a, i, lane);
    // Tiles per row, and their cost for the aligned split: a sequence with n > 0
    // tiles costs kTileCost n + kPieceCost (opening and closing a piece takes time
    // beyond its tiles).
    constexpr int pcost = kPieceCost;
    int mine_t = 0, mine_w = 0;
#pragma unroll 4
    for (int i = lane; i < S; i += kWave) {
        const int n = tiles_of(ctx_of(a, i));
        mine_t += n;
        mine_w += n > 0 ? kTileCost * n + pcost : 0;
    }
    int T_row = uni(wave_sum(mine_t));
    int W_row = uni(wave_sum(mine_w));
    if constexpr (NW > 1) {
        // One count for the whole workgroup: its waves then run the same number of
        // tiles and meet the per-tile barrier equally often, even if the lengths
        // were changed while the kernel ran.
        __shared__ int s_tw[2];
        if (threadIdx.x == 0) {
            s_tw[0] = T_row;
            s_tw[1] = W_row;
        }
        __syncthreads();
        T_row = s_tw[0];
        W_row = s_tw[1];
    }
    // Per-head path: whether the workgroup's rows meet at every tile (below); the
    // same for every wave of the workgroup, since T_row is.
    const bool tile_barrier = !Stream || T_row >= kBarrierTilesPerSeq * static_cast<long long>(S);
    int32_t* rec = a.unit_rec + static_cast<size_t>(u) * kRecInts;
    if (lane == 0) rec[0] = -1;  // set below when a split sequence ends in this unit
    // The unit's tiles: n_tiles from tile tin of row row0, starting in sequence seq0 at
    // its tile t00.  first_*: units holding the first and last tile of the sequence the
    // unit's first piece belongs to, when that piece starts inside it (else -1);
    // last_*: the same for the last piece, when it runs past the unit's end.
    int n_tiles = 0, row0 = 0, tin = 0, seq0 = 0, t00 = 0;
    int C = 0, start = 0;  // one-line split
    int first_us = -1, first_ue = -1, last_us = -1, last_ue = -1;
    if (a.aligned) {
        // Every row is cut into the same Wr ranges of CC cost units; range k covers
        // the tiles whose cost starts at or after k CC and before (k + 1) CC.  The tile
        // at cost b, in sequence i with cost prefix P_i, tile prefix S_i and n_i tiles,
        // is S_i + clamp(ceil((b - P_i - kPieceCost) / kTileCost), 0, n_i); tile t of
        // sequence i lies in range floor((P_i + kPieceCost + kTileCost t) / CC).
        // CC >= kTileCost: consecutive tiles of a sequence start kTileCost apart, so
        // every range strictly between a split sequence's first and last range holds
        // a tile of it, and the merge finds a piece in every unit from us to ue.
        row0 = u / Wr;
        const int k = u - row0 * Wr;
        const int CC = max(kTileCost, (W_row + Wr - 1) / Wr);
        const int b0 = k * CC;
        const int b1 = min(b0 + CC, W_row);
        if (u < Wrun && b0 < W_row) {
            int tb0 = -1, tb1 = b1 >= W_row ? T_row : -1;
            int carry_t = 0, carry_w = 0;
            for (int base = 0; base < S && (tb0 < 0 || tb1 < 0); base += kWave) {
                const int i = base + lane;
                const int n = i < S ? tiles_of(ctx_of(a, i)) : 0;
                const int w = n > 0 ? kTileCost * n + pcost : 0;
                const int incl_t = wave_inclusive_scan(n, lane) + carry_t;
                const int incl_w = wave_inclusive_scan(w, lane) + carry_w;
                auto locate = [&](int b, int& tb, int& seq, int& t, int& us, int& ue) {
                    const unsigned long long hit = __ballot(incl_w > b);
                    if (!hit) return;
                    const int f = __ffsll(static_cast<long long>(hit)) - 1;
                    const int nf = __builtin_amdgcn_readlane(n, f);
                    const int pf_ = __builtin_amdgcn_readlane(incl_w - w, f);
                    const int x = b - pf_ - pcost;
                    t = min(x <= 0 ? 0 : (x + kTileCost - 1) / kTileCost, nf);
                    tb = __builtin_amdgcn_readlane(incl_t - n, f) + t;
                    seq = base + f;
                    if (t > 0 && t < nf) {  // the boundary cuts sequence seq
                        us = row0 * Wr + (pf_ + pcost) / CC;
                        ue = row0 * Wr + (pf_ + pcost + kTileCost * (nf - 1)) / CC;
                    }
                };
                int s_unused = 0, t_unused = 0;
                if (tb0 < 0) locate(b0, tb0, seq0, t00, first_us, first_ue);
                if (tb1 < 0) locate(b1, tb1, s_unused, t_unused, last_us, last_ue);
                carry_t = __builtin_amdgcn_readlane(incl_t, kWave - 1);
                carry_w = __builtin_amdgcn_readlane(incl_w, kWave - 1);
            }
            tin = tb0;
            n_tiles = tb0 >= 0 && tb1 >= 0 ? tb1 - tb0 : 0;
        }
        first_us = uni(first_us);
        first_ue = uni(first_ue);
        last_us = uni(last_us);
        last_ue = uni(last_ue);
    } else {
        const int total = R * T_row;
        C = (total + W - 1) / W;
        start = u * C;
        n_tiles = min(start + C, total) - start;
        row0 = T_row > 0 ? start / T_row : 0;
        tin = start - row0 * T_row;
        if (n_tiles > 0) {
            // Find the sequence holding tile `tin` of the row.
            int carry = 0;
            for (int base = 0; base < S; base += kWave) {
                const int i = base + lane;
                const int n = i < S ? tiles_of(ctx_of(a, i)) : 0;
                const int incl = wave_inclusive_scan(n, lane) + carry;
                const unsigned long long hit = __ballot(incl > tin);
                if (hit) {
                    const int f = __ffsll(static_cast<long long>(hit)) - 1;
                    seq0 = base + f;
                    t00 = tin - __shfl(incl - n, f);
                    break;
                }
                carry = __shfl(incl, kWave - 1);
            }
        }
    }
    if (T_row == 0 || n_tiles <= 0) return;

    const u32x4* kc = static_cast<const u32x4*>(a.k_cache);
    const u32x4* vc = static_cast<const u32x4*>(a.v_cache);

    // ---- fetch side: chunk, next lane of it, tiles issued so far
    Chunk ch = build_chunk<Path, Step, Half>(a, Cursor{row0, uni(seq0), uni(t00)}, n_tiles, lane);
    int kf = 0, fetched = 0;
    int f_seq = -1, f_row = -1;  // piece of the last fetched tile
    typename Path::Q q, qn;

    struct Buf {
        u32x4 k[NL], v[NL];
        TileRef r;
        bool opens;  // first tile of a piece
        TokenV<T, NL> tok;    // decode step: the new token's V values, when the tile holds its place
        bool pend;            // decode step: the tile's write-back is still to be stored
    };
    Buf A, B;
    A.pend = B.pend = false;

    // A split sequence's pieces sit in units us .. ue (in unit us in record slot 1,
    // elsewhere in slot 0).  With the merge folded in (a.fused), each holder
    // counts its arrival on the count of unit ue once its record is written; `old` (lane 0)
    // is the count before it.  The holder that finds the other ue - us pieces there
    // merges them and sets the count back to zero for the next call.
    struct Split {
        int old, us, ue, row, seq;
    };
    Split first_split{};
    bool has_first = false;
    bool arrive_first = false;  // first_split's record written, its count not yet moved
    // Count the first piece's arrival; every load and store of the wave has completed
    // (the caller has just waited), so its record is visible.
    auto arrive = [&]() {
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0)
            first_split.old = __hip_atomic_fetch_add(a.split_count_end - 1 - first_split.ue, 1,
                                                     __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        arrive_first = false;
    };
    // Decode step: a tile of a sequence's last block takes the new token at its place
    // (fixup, before the tile is folded).  When the block is copied (copy-on-write) the
    // whole tile is written to the copy, and the wave holding the token's tile also
    // copies the block's tiles after it; a block written in place needs nothing more
    // (the token itself was scattered at the start).  The write-back (flush) waits
    // until the buffer is reused, right after the next wait for loads, so that its
    // stores complete alongside the next tile's loads.
    u32x4* const kw = const_cast<u32x4*>(static_cast<const u32x4*>(a.k_cache));
    u32x4* const vw = const_cast<u32x4*>(static_cast<const u32x4*>(a.v_cache));
    // Half: the register layout of a 16-token tile is unchanged, but tokens 0..7 come
    // from the first block's 8-token tile and tokens 8..15 from the second's.  Lane
    // l = 16 j + i reads K load s (token i, dim chunk 4 s + j) at (4 s + j) 8 + i % 8 of
    // block i / 8, and V load m (tokens 4 j .. 4 j + 3) at (2 m + j % 2) 16 + i of block
    // j / 2: per lane a block choice, an offset, and a stride of 32 groups per load.
    constexpr int HALF_U4 = Path::TILE_U4 / 2;
    const int k_lane = 8 * (lane >> 4) + (lane & 7);
    const int v_lane = 16 * ((lane >> 4) & 1) + (lane & 15);
    const bool k_hi = (lane & 15) >= 8;
    const bool v_hi = (lane >> 4) >= 2;
    auto flush = [&](Buf& b) {
        if constexpr (Step && Half) {
            // copy-on-write of an 8-token block: the lanes holding the token's block
            // write it whole to the copy (blocks after it do not exist in the tile)
            if (!b.pend) return;
            b.pend = false;
            const bool hi = b.r.ptok >= 8;
            const size_t wo = static_cast<size_t>(b.r.wtoff) * HALF_U4;
            if (k_hi == hi) {
#pragma unroll
                for (int s = 0; s < NL; ++s) kw[wo + k_lane + 32 * s] = b.k[s];
            }
            if (v_hi == hi) {
#pragma unroll
                for (int s = 0; s < NL; ++s) vw[wo + v_lane + 32 * s] = b.v[s];
            }
        } else if constexpr (Step) {
            if (!b.pend) return;
            b.pend = false;
            const int p = b.r.ptok;
            const size_t wo = static_cast<size_t>(b.r.wtoff) * Path::TILE_U4;
#pragma unroll
            for (int s = 0; s < NL; ++s) kw[wo + lane + s * kWave] = b.k[s];
#pragma unroll
            for (int s = 0; s < NL; ++s) vw[wo + lane + s * kWave] = b.v[s];
            if (p >= 0) {
                const int tpb = a.tiles_per_block;
                const int tib = b.r.tile % tpb;
                for (int tt = tib + 1; tt < tpb; ++tt) {
                    const size_t so = static_cast<size_t>(b.r.toff + (tt - tib) * a.num_kv_heads) * Path::TILE_U4;
                    const size_t dof = static_cast<size_t>(b.r.wtoff + (tt - tib) * a.num_kv_heads) * Path::TILE_U4;
                    // a rare path (the tiles past the token of a copied block): one group at a time
#pragma unroll 1
                    for (int s = 0; s < NL; ++s) {
                        const u32x4 ck = kc[so + lane + s * kWave];
                        const u32x4 cv = vc[so + lane + s * kWave];
                        kw[dof + lane + s * kWave] = ck;
                        vw[dof + lane + s * kWave] = cv;
                    }
                }
            }
        }
    };
    auto fixup = [&](Buf& b) {
        if constexpr (Step) {
            if (b.r.wtoff < 0) return;
            if (b.r.ptok >= 0) patch_token_v<T, NL>(b.v, b.tok, b.r.ptok, lane);
            // copy-on-write: the tile (8-token blocks: the token's block) goes to the copy
            b.pend = b.r.wtoff != (Half && b.r.ptok >= 8 ? b.r.toff2 : b.r.toff);
        }
    };
    auto issue = [&](Buf& b) {
        // One tile in flight per wave: the previous tile's loads have all returned
        // before the next tile is requested.  Measured on MI355X, this sustains more
        // HBM bandwidth than keeping two tiles in flight (the extra requests only
        // lengthen the memory queues); the unit count then sets the bytes in flight.
        wait_all_loads();
        if (arrive_first) arrive();
        // Decode step: this buffer's write-back goes out now, beside the next tile's
        // loads, so that no wait is spent on it alone.
        if constexpr (Step) flush(b);
        // The rows of a workgroup walk the same tiles; meeting once per tile keeps
        // their requests for one block's adjacent heads (consecutive 4 KiB pieces of
        // K and of V) reaching memory together.  Measured with streamed loads, that
        // pays for the per-head path on long sequences (G = 1: 344 against 353 us on
        // a batch of 64 32-head sequences of 2112 tokens on average) but not on many
        // short ones, whose ranges cross many sequence ends (1079 against 1089 us of
        // attention per step without it over about 690 40-head sequences of about 600
        // tokens), so with streamed loads the per-head path meets only when the batch
        // averages kBarrierTilesPerSeq tiles or more per sequence.  With cached loads
        // (blocks shared between sequences) it always meets: on a prefix-cached
        // serving trace of sequences as short, 1135 against 1176 us of attention per
        // step with it.  The group path never meets (G = 4: 220 us without it against
        // 221 with it on a batch of 256).
        if constexpr (NW > 1 && Path::GH == 1) {
            if (tile_barrier) __syncthreads();
        }
        while (kf == ch.n) {  // chunk used up: describe the next tiles (empty chunks only
                              // arise from runs of sequences with no cached tokens)
            if (ch.next.row >= a.rows) {
                // The walk ran past the last row, which only happens if context_lens
                // changed under the kernel: fold harmless in-pool tiles instead of spinning.
                ch.n = 1;
                ch.seq = ch.tile = ch.row = ch.ctx = ch.toff = ch.toff2 = 0;
                ch.wtoff = ch.ptok = -1;
                kf = 0;
                break;
            }
            ch = build_chunk<Path, Step, Half>(a, ch.next, n_tiles - fetched, lane);
            kf = 0;
        }
        b.r = tile_ref<Step, Half>(ch, kf);
        ++kf;
        ++fetched;
        // The query of a new piece is requested before the tile, so that waiting
        // for it never waits for the tile's loads as well.
        b.opens = (b.r.seq != f_seq) || (b.r.row != f_row);
        if (b.opens) Path::load_q(a, qn, b.r.row, b.r.seq, lane);
        f_seq = b.r.seq;
        f_row = b.r.row;
        // Uniform tile base (scalar registers) + lane offset: one contiguous KiB per load.
        // A tile of private context is read once per call: non-temporal loads stream it
        // past the caches instead of filling them with lines nobody reads again.
        // Blocks shared between sequences are re-read within the call, so the caller
        // can keep them cached instead (ordinary loads).
        const size_t off = static_cast<size_t>(b.r.toff) * (Half ? HALF_U4 : Path::TILE_U4);
        const u32x4* kt = kc + off;
        const u32x4* vt = vc + off;
        // Half: this lane's first group of K and of V (loads 32 groups apart)
        const u32x4* kh = kc + static_cast<size_t>(k_hi ? b.r.toff2 : b.r.toff) * HALF_U4 + k_lane;
        const u32x4* vh = vc + static_cast<size_t>(v_hi ? b.r.toff2 : b.r.toff) * HALF_U4 + v_lane;
        if constexpr (Step) {
            // Every lane reads its V values of the new token (harmless ones when it has
            // none), so the loads in flight never depend on the tile.
            const size_t ro = (static_cast<size_t>(b.r.seq) * a.num_kv_heads +
                               Path::kv_head(a, b.r.row)) * D;
            const T* vnew = static_cast<const T*>(a.v_new);
            load_token_v<T, NL>(b.tok, vnew + ro, vnew, b.r.ptok, lane);
            if (Half && b.r.ptok >= 0) {
                // As below, with the two blocks' addressing.
                constexpr int X = TokenV<T, NL>::X;
                const T* krow = static_cast<const T*>(a.k_new) + ro + (lane >> 4) * X;
                const bool mine = (lane & 15) == b.r.ptok;
                const u32x4* kp = mine ? reinterpret_cast<const u32x4*>(krow) : kh;
                const int ks = mine ? 4 * X * static_cast<int>(sizeof(T)) / 16 : 32;
#pragma unroll
                for (int s = 0; s < NL; ++s) b.k[s] = kp[s * ks];
#pragma unroll
                for (int s = 0; s < NL; ++s) b.v[s] = vh[32 * s];
                return;
            }
            if (!Half && b.r.ptok >= 0) {
                // The new token's tile: this launch has already written the token into
                // it (the scatter at the start), and non-temporal loads of lines written
                // in the same launch were measured to cost ~17 us per step on the
                // batch-256 config, so this tile is read with ordinary loads.  The lanes
                // holding the token's place read its K groups from the new row instead
                // (the scatter's bytes may sit in another XCD's cache).
                constexpr int X = TokenV<T, NL>::X;
                const T* krow = static_cast<const T*>(a.k_new) + ro + (lane >> 4) * X;
                const bool mine = (lane & 15) == b.r.ptok;
                const u32x4* kp = mine ? reinterpret_cast<const u32x4*>(krow) : kt + lane;
                const int ks = mine ? 4 * X * static_cast<int>(sizeof(T)) / 16 : kWave;
#pragma unroll
                for (int s = 0; s < NL; ++s) b.k[s] = kp[s * ks];
                const __amdgpu_buffer_rsrc_t vr = __builtin_amdgcn_make_buffer_rsrc(
                    const_cast<u32x4*>(vt), static_cast<short>(0), Path::TILE_U4 * 16, kBufferRsrcWord3);
#pragma unroll
                for (int s = 0; s < NL; ++s)
                    b.v[s] = __builtin_amdgcn_raw_buffer_load_b128(vr, (lane + s * kWave) * 16, 0, 0);
                return;
            }
        }
        if constexpr (Half) {
            if constexpr (!Stream) {
#pragma unroll
                for (int s = 0; s < NL; ++s) b.k[s] = kh[32 * s];
#pragma unroll
                for (int s = 0; s < NL; ++s) b.v[s] = vh[32 * s];
            } else {
#pragma unroll
                for (int s = 0; s < NL; ++s) b.k[s] = __builtin_nontemporal_load(kh + 32 * s);
#pragma unroll
                for (int s = 0; s < NL; ++s) b.v[s] = __builtin_nontemporal_load(vh + 32 * s);
            }
        } else if constexpr (!Stream) {
#pragma unroll
            for (int s = 0; s < NL; ++s) b.k[s] = kt[lane + s * kWave];
#pragma unroll
            for (int s = 0; s < NL; ++s) b.v[s] = vt[lane + s * kWave];
        } else {
#pragma unroll
            for (int s = 0; s < NL; ++s) b.k[s] = __builtin_nontemporal_load(kt + lane + s * kWave);
#pragma unroll
            for (int s = 0; s < NL; ++s) b.v[s] = __builtin_nontemporal_load(vt + lane + s * kWave);
        }
    };


    // ---- compute side: the open piece
    typename Path::Acc st;
    int p_seq = -1, p_row = 0, p_t0 = 0, p_last = 0, p_ctx = 0, p_g0 = 0, npieces = 0;
    auto close_piece = [&](Split& sp, bool defer) -> bool {
        const int nts = tiles_of(p_ctx);
        const bool whole = (p_t0 == 0) && (p_last == nts - 1);
        // A split piece's record goes to slot 1 when it holds its sequence's first
        // tile (it is then its unit's last piece), else to slot 0 (its unit's first).
        const int slot = p_t0 == 0 ? 1 : 0;
        float* prec = a.pieces + (static_cast<size_t>(u) * 2 + slot) * pf;
        Path::finish(a, st, p_row, p_seq, whole, prec, lane);
        ++npieces;
        if (whole) return false;
        if (a.aligned) {
            // only the first piece can start inside its sequence, only the last run on
            sp.us = p_t0 > 0 ? first_us : last_us;
            sp.ue = p_t0 > 0 ? first_ue : last_ue;
        } else {
            const int seq_begin = start + p_g0 - p_t0;
            sp.us = seq_begin / C;
            sp.ue = (seq_begin + nts - 1) / C;
        }
        // Units outside [0, Wrun) only arise if the lengths changed under the kernel:
        // leave that split unmerged rather than address records that do not exist.
        if (sp.us < 0 || sp.ue < sp.us || sp.ue >= Wrun) return false;
        sp.row = p_row;
        sp.seq = p_seq;
        sp.old = 0;
        // For the two-kernel path: the split that ends in this unit is merged by it.
        if (p_t0 > 0 && sp.ue == u && lane == 0) {
            rec[0] = p_row;
            rec[1] = p_seq;
            rec[2] = sp.us;
            rec[3] = sp.ue;
        }
        if (!a.fused) return false;
        if (defer) return true;  // counted after the next tile's wait (arrive below)
        // The record's device-scope stores are complete before the count moves.
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        wait_all_loads();
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        if (lane == 0)
            sp.old = __hip_atomic_fetch_add(a.split_count_end - 1 - sp.ue, 1, __ATOMIC_RELAXED,
                                            __HIP_MEMORY_SCOPE_AGENT);
        return true;
    };
    auto merge_if_last = [&](const Split& sp) {
        if (__builtin_amdgcn_readfirstlane(sp.old) != sp.ue - sp.us) return;
        __atomic_signal_fence(__ATOMIC_SEQ_CST);
        merge_pieces<T, D, Path::GH>(a, sp.row, sp.seq, sp.us, sp.ue, lane);
        if (lane == 0)
            __hip_atomic_store(a.split_count_end - 1 - sp.ue, 0, __ATOMIC_RELAXED,
                               __HIP_MEMORY_SCOPE_AGENT);
    };
    auto enter = [&](const Buf& b, int g) {
        if (b.opens) {
            // Only a unit's first piece can close inside the loop as a split one (it
            // began in an earlier unit); its merge waits until the tiles are done.
            if (p_seq >= 0 && close_piece(first_split, true)) {
                has_first = true;
                arrive_first = true;
            }
#pragma unroll
            for (int s = 0; s < NL; ++s) q.v[s] = qn.v[s];
            Path::reset(st);
            p_seq = b.r.seq;
            p_row = b.r.row;
            p_t0 = b.r.tile;
            p_ctx = b.r.ctx;
            p_g0 = g;
        }
        p_last = b.r.tile;
    };

    // Steady state: every trip folds two tiles and issues the two after them.  The
    // issues are unconditional inside the loop (the last tiles are peeled off below):
    // a conditional issue would join paths with different numbers of loads in
    // flight, and the compiler then waits for all of them before the MFMAs.
    issue(A);
    int g = 0;
    for (; g + 2 < n_tiles; g += 2) {
        enter(A, g);
        issue(B);
        fixup(A);
        Path::tile(a, st, q, A.k, A.v, A.r.tile, A.r.ctx, lane);
        enter(B, g + 1);
        issue(A);
        fixup(B);
        Path::tile(a, st, q, B.k, B.v, B.r.tile, B.r.ctx, lane);
    }
    enter(A, g);
    if (g + 1 < n_tiles) {
        issue(B);
        fixup(A);
        Path::tile(a, st, q, A.k, A.v, A.r.tile, A.r.ctx, lane);
        enter(B, g + 1);
        fixup(B);
        Path::tile(a, st, q, B.k, B.v, B.r.tile, B.r.ctx, lane);
    } else {
        fixup(A);
        Path::tile(a, st, q, A.k, A.v, A.r.tile, A.r.ctx, lane);
    }
    flush(A);
    flush(B);
    if (arrive_first) {
        wait_all_loads();
        arrive();
    }
    Split last_split{};
    const bool has_last = close_piece(last_split, false);
    if (has_first) merge_if_last(first_split);
    if (has_last) merge_if_last(last_split);
}

// ---------------------------------------------------------------------------------
// Pass 2 (separate kernel): unit u merges the split sequence whose last piece it
// holds (its first piece, when that sequence began in an earlier unit and ends
// inside unit u).
template <typename T, int D, int GH>
__global__ __launch_bounds__(64) void decode_pass2(DecodeArgs a) {
    const int lane = threadIdx.x;
    const int u = blockIdx.x;
    if (a.aligned && u >= (a.num_units / a.rows) * a.rows) return;  // never ran pass 1
    const int32_t* rec = a.unit_rec + static_cast<size_t>(u) * kRecInts;
    const int row = rec[0];
    if (row < 0) return;
    const int seq = rec[1], us = rec[2], ue = rec[3];
    if (seq < 0 || seq >= a.num_seqs || row >= a.rows || ue != u || us < 0 || us >= u) return;
    merge_pieces<T, D, GH>(a, row, seq, us, u, lane);
}

template <typename T, int D>
hipError_t launch_pass2(const DecodeArgs& a, hipStream_t st) {
    const dim3 grid(a.num_units), block(kWave);
    switch (a.heads_per_row) {
        case 1: hipLaunchKernelGGL((decode_pass2<T, D, 1>), grid, block, 0, st, a); break;
        case 2: hipLaunchKernelGGL((decode_pass2<T, D, 2>), grid, block, 0, st, a); break;
        case 4: hipLaunchKernelGGL((decode_pass2<T, D, 4>), grid, block, 0, st, a); break;
        case 8: hipLaunchKernelGGL((decode_pass2<T, D, 8>), grid, block, 0, st, a); break;
        case 16: hipLaunchKernelGGL((decode_pass2<T, D, 16>), grid, block, 0, st, a); break;
        default: return hipErrorInvalidValue;
    }
    return hipGetLastError();
}

template <class Path, typename T, int D, int NW, bool Stream, bool Step, bool Half>
hipError_t launch_pass1_nw(const DecodeArgs& a, int groups, hipStream_t st) {
    // (a cooperative launch would guarantee residency outright, but measured ~15 us
    // slower per launch on this part; dispatch in index order is what the step's
    // wait relies on)
    hipLaunchKernelGGL((decode_pass1<Path, T, D, NW, Stream, Step, Half>), dim3(groups),
                       dim3(NW * kWave), 0, st, a);
    return hipSuccess;
}

template <class Path, typename T, int D, bool Stream, bool Step, bool Half>
hipError_t launch_pass1(const DecodeArgs& a, int nw, int groups, hipStream_t st) {
    switch (nw) {
        case 1: return launch_pass1_nw<Path, T, D, 1, Stream, Step, Half>(a, groups, st);
        case 2: return launch_pass1_nw<Path, T, D, 2, Stream, Step, Half>(a, groups, st);
        case 4: return launch_pass1_nw<Path, T, D, 4, Stream, Step, Half>(a, groups, st);
        case 8: return launch_pass1_nw<Path, T, D, 8, Stream, Step, Half>(a, groups, st);
        default: return hipErrorInvalidValue;
    }
}

// Step: one launch with the step's writes, merge folded in.  Otherwise pass 1 (bit 0
// of passes) and, when the merge is not folded in, pass 2 (bit 1).
template <class Path, typename T, int D, bool Stream, bool Step, bool Half>
hipError_t launch_two_pass(const DecodeArgs& a, int passes, hipStream_t st) {
    const int nw = a.waves_per_group;
    const int groups = nw > 1 ? (a.num_units / a.rows) * a.rows / nw : a.num_units;
    if (Step || (passes & 1)) {
        const hipError_t e0 = launch_pass1<Path, T, D, Stream, Step, Half>(a, nw, groups, st);
        if (e0 != hipSuccess) return e0;
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess || Step) return e;
    }
    if ((passes & 2) && !a.fused) {
        hipLaunchKernelGGL((decode_pass2<T, D, Path::GH>), dim3(a.num_units), dim3(kWave), 0, st, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

template <int D, bool Stream, bool Step, bool Half>
hipError_t launch_group(const DecodeArgs& a, int passes, hipStream_t st) {
    switch (a.group) {
        case 2: return launch_two_pass<GroupPath<D, 2>, uint16_t, D, Stream, Step, Half>(a, passes, st);
        case 4: return launch_two_pass<GroupPath<D, 4>, uint16_t, D, Stream, Step, Half>(a, passes, st);
        case 8: return launch_two_pass<GroupPath<D, 8>, uint16_t, D, Stream, Step, Half>(a, passes, st);
        case 16: return launch_two_pass<GroupPath<D, 16>, uint16_t, D, Stream, Step, Half>(a, passes, st);
        default: return hipErrorInvalidValue;
    }
}

}  // namespace

template <bool Stream, bool Step, bool Half>
hipError_t launch_decode_variant(int dtype, int head_dim, bool use_group_kernel, const DecodeArgs& a,
                                 int passes, hipStream_t stream) {
    if (dtype == 1) {  // bf16
        if (use_group_kernel) {
            if (head_dim == 128) return launch_group<128, Stream, Step, Half>(a, passes, stream);
            if (head_dim == 64) return launch_group<64, Stream, Step, Half>(a, passes, stream);
        } else {
            if (head_dim == 128)
                return launch_two_pass<HeadPath<uint16_t, 128>, uint16_t, 128, Stream, Step, Half>(a, passes, stream);
            if (head_dim == 64)
                return launch_two_pass<HeadPath<uint16_t, 64>, uint16_t, 64, Stream, Step, Half>(a, passes, stream);
        }
    } else if (dtype == 0 && !use_group_kernel) {
        if (head_dim == 128)
            return launch_two_pass<HeadPath<uint32_t, 128>, uint32_t, 128, Stream, Step, Half>(a, passes, stream);
        if (head_dim == 64)
            return launch_two_pass<HeadPath<uint32_t, 64>, uint32_t, 64, Stream, Step, Half>(a, passes, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
