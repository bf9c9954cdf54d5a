// Paged decode attention for gfx950: pass 1 (block-table gather, QK^T, online
// softmax, PV) and pass 2 (log-sum-exp merge of split sequences).
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
// end, rows one after another, and the whole line is cut into num_units equal
// ranges.  One wavefront owns one range: perfectly even work whatever the
// length mix.  A sequence that a range holds whole is finished in place; a
// sequence cut by range ends leaves partial (max, sum, accumulator) records,
// and pass 2 merges them with the log-sum-exp rule.  Every wave scans the
// context lengths itself to find its range, so no planning kernel runs first.
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

#include "pagedkv_internal.h"

namespace pkv {
namespace {

typedef unsigned u32x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((__vector_size__(4 * sizeof(float))));
typedef __bf16 bf16x8 __attribute__((__vector_size__(8 * sizeof(__bf16))));
typedef __bf16 bf16x2 __attribute__((__vector_size__(2 * sizeof(__bf16))));
typedef short s16x4 __attribute__((__vector_size__(4 * sizeof(short))));

constexpr float kNegInf = -__builtin_inff();

__device__ __forceinline__ int uni(int x) { return __builtin_amdgcn_readfirstlane(x); }

// Reinterpret one 32-bit word as two bf16.  The word is taken by value on purpose:
// clang's __builtin_bit_cast applied directly to an ext-vector element reads
// element 0 whatever the index, so vector elements must be copied out first.
__device__ __forceinline__ bf16x2 as_bf16x2(uint32_t w) { return __builtin_bit_cast(bf16x2, w); }

__device__ __forceinline__ float bf_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf_hi(uint32_t w) { return __uint_as_float(w & 0xffff0000u); }

// Round a finite non-negative float to bf16, nearest-even (softmax weights).
__device__ __forceinline__ uint32_t bf16_rne_finite(float f) {
    const uint32_t u = __float_as_uint(f);
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}

// Round any float to bf16, nearest-even; NaN stays NaN.
__device__ __forceinline__ uint16_t bf16_rne(float f) {
    const uint32_t u = __float_as_uint(f);
    if ((u & 0x7fffffffu) > 0x7f800000u) return static_cast<uint16_t>((u >> 16) | 0x40u);
    return static_cast<uint16_t>((u + 0x7fffu + ((u >> 16) & 1u)) >> 16);
}

__device__ __forceinline__ float fast_exp2(float x) { return __builtin_amdgcn_exp2f(x); }

__device__ __forceinline__ int wave_sum(int v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o);
    return v;
}

__device__ __forceinline__ int wave_inclusive_scan(int v, int lane) {
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
        const int t = __shfl_up(v, o);
        if (lane >= o) v += t;
    }
    return v;
}

// Context length of sequence i, clamped to what its table row can address.
__device__ __forceinline__ int ctx_of(const DecodeArgs& a, int i) {
    const int cap = a.max_blocks * a.tiles_per_block * kTile;
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

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) { *p = bf16_rne(x); }
template <>
__device__ __forceinline__ void store_out<uint32_t>(uint32_t* p, float x) {
    *p = __float_as_uint(x);
}

// Zero every query head of sequence `seq` (a sequence with no cached tokens).
template <typename T, int D>
__device__ void write_zero_seq(const DecodeArgs& a, int seq, int lane) {
    T* o = static_cast<T*>(a.out) + static_cast<size_t>(seq) * a.num_q_heads * D;
    for (int k = lane; k < a.num_q_heads * D; k += kWave) o[k] = 0;
}

// ---------------------------------------------------------------------------------
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

    static __device__ int piece_floats() { return (D + 2 + 3) & ~3; }

    struct State {
        u32x4 q[NL];
        float m, l;
        float acc[NL][E];
    };

    static __device__ __forceinline__ void tile(const DecodeArgs& a, State& st, const u32x4* kb,
                                                const u32x4* vb, int t, int ctx, int lane) {
        const int j = lane >> 4, i = lane & 15;
        // QK: partial dot over this lane's dims, then across the four rows.
        float part = 0.f;
#pragma unroll
        for (int s = 0; s < NL; ++s) {
#pragma unroll
            for (int w = 0; w < 4; ++w) {
                if constexpr (kBf16) {
                    part = __builtin_amdgcn_fdot2_f32_bf16(as_bf16x2(kb[s][w]),
                                                           as_bf16x2(st.q[s][w]), part, false);
                } else {
                    part = __builtin_fmaf(__uint_as_float(kb[s][w]), __uint_as_float(st.q[s][w]),
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

    template <bool kWhole>
    static __device__ void finish(const DecodeArgs& a, State& st, int qh, int seq, float* rec,
                                  int lane) {
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
        if constexpr (kWhole) {
            T* o = static_cast<T*>(a.out) + (static_cast<size_t>(seq) * a.num_q_heads + qh) * D;
            const float inv = 1.f / L;
#pragma unroll
            for (int mm = 0; mm < NL; ++mm)
#pragma unroll
                for (int e = 0; e < E; ++e) store_out<T>(o + 16 * E * mm + 16 * e + i, st.acc[mm][e] * inv);
        } else {
#pragma unroll
            for (int mm = 0; mm < NL; ++mm)
#pragma unroll
                for (int e = 0; e < E; ++e) rec[16 * E * mm + 16 * e + i] = st.acc[mm][e];
            if (i == 0) {
                rec[D] = st.m;
                rec[D + 1] = L;
            }
        }
    }

    static __device__ void piece(const DecodeArgs& a, int row, int seq, int t0, int t1, bool whole,
                                 float* rec, int lane) {
        const int qh = row;
        const int kvh = qh / a.group;
        const int j = lane >> 4;
        const int ctx = ctx_of(a, seq);
        State st;
        const T* qrow = static_cast<const T*>(a.q) + (static_cast<size_t>(seq) * a.num_q_heads + qh) * D;
#pragma unroll
        for (int s = 0; s < NL; ++s) st.q[s] = *reinterpret_cast<const u32x4*>(qrow + (4 * s + j) * X);
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int mm = 0; mm < NL; ++mm)
#pragma unroll
            for (int e = 0; e < E; ++e) st.acc[mm][e] = 0.f;
        run_tiles(a, st, seq, kvh, t0, t1, ctx, lane);
        if (whole)
            finish<true>(a, st, qh, seq, rec, lane);
        else
            finish<false>(a, st, qh, seq, rec, lane);
    }

    static __device__ void run_tiles(const DecodeArgs& a, State& st, int seq, int kvh, int t0,
                                     int t1, int ctx, int lane);
};

// ---------------------------------------------------------------------------------
// Group path (MFMA, bf16).  Lane l = 16 j + i; query column i holds head i % G.
//   K load s: token i, dims 32 s + 8 j + x  -> A operand of S = K Q^T (16x16x32)
//   S[r]    : token 4 j + r, head column i  -> B operand of O^T = V^T P^T (16x16x16)
//   V load m: tokens 4j .. 4j+3 of dims 32 m + i (words 0,1) and 32 m + 16 + i (words 2,3)
//             -> A operands of the two 16-dim groups 2m, 2m+1
//   acc[g][r]: dim 16 g + 4 j + r, head column i
template <int D>
struct GroupPath {
    using T = uint16_t;
    static constexpr int NL = D / 32;  // 16-B loads per lane per tile (K and V)
    static constexpr int NG = D / 16;  // 16-dim output groups
    static constexpr int TILE_U4 = D * 2;

    struct State {
        u32x4 q[NL];
        float m, l;
        f32x4 acc[NG];
    };

    static __device__ __forceinline__ void tile(const DecodeArgs& a, State& st, const u32x4* kb,
                                                const u32x4* vb, int t, int ctx, int lane) {
        const int j = lane >> 4;
        f32x4 S = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int s = 0; s < NL; ++s)
            S = __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, kb[s]),
                                                        __builtin_bit_cast(bf16x8, st.q[s]), S, 0,
                                                        0, 0);
        const int tok0 = t * kTile + 4 * j;
        float sc[4];
#pragma unroll
        for (int r = 0; r < 4; ++r) sc[r] = (tok0 + r < ctx) ? S[r] * a.scale_log2e : kNegInf;
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
        const bool last = t * kTile + kTile > ctx;
        uint32_t mask01 = 0xffffffffu, mask23 = 0xffffffffu;
        if (last) {
            const int nv = ctx - tok0;
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

    static __device__ void piece(const DecodeArgs& a, int row, int seq, int t0, int t1, bool whole,
                                 float* rec, int lane) {
        const int kvh = row;
        const int G = a.group;
        const int j = lane >> 4, i = lane & 15;
        const int ctx = ctx_of(a, seq);
        State st;
        const T* qrow = static_cast<const T*>(a.q) +
                        (static_cast<size_t>(seq) * a.num_q_heads + kvh * G + (i % G)) * D;
#pragma unroll
        for (int s = 0; s < NL; ++s) st.q[s] = *reinterpret_cast<const u32x4*>(qrow + 32 * s + 8 * j);
        st.m = kNegInf;
        st.l = 0.f;
#pragma unroll
        for (int g = 0; g < NG; ++g) st.acc[g] = (f32x4){0.f, 0.f, 0.f, 0.f};
        run_tiles(a, st, seq, kvh, t0, t1, ctx, lane);
        // finish
        float L = st.l;
        L += __shfl_xor(L, 16);
        L += __shfl_xor(L, 32);
        if (i >= G) return;
        if (whole) {
            T* o = static_cast<T*>(a.out) + (static_cast<size_t>(seq) * a.num_q_heads + kvh * G + i) * D;
            const float inv = 1.f / L;
#pragma unroll
            for (int g = 0; g < NG; ++g) {
                const uint32_t lo = bf16_rne(st.acc[g][0] * inv) | (uint32_t(bf16_rne(st.acc[g][1] * inv)) << 16);
                const uint32_t hi = bf16_rne(st.acc[g][2] * inv) | (uint32_t(bf16_rne(st.acc[g][3] * inv)) << 16);
                *reinterpret_cast<uint2*>(o + 16 * g + 4 * j) = make_uint2(lo, hi);
            }
        } else {
#pragma unroll
            for (int g = 0; g < NG; ++g)
                *reinterpret_cast<f32x4*>(rec + i * D + 16 * g + 4 * j) = st.acc[g];
            if (j == 0) {
                rec[G * D + i] = st.m;
                rec[G * D + G + i] = L;
            }
        }
    }

    static __device__ void run_tiles(const DecodeArgs& a, State& st, int seq, int kvh, int t0,
                                     int t1, int ctx, int lane);
};

// ---------------------------------------------------------------------------------
// The tile loop shared by both paths: gather through the block table with the
// next tile's loads in flight while the current tile is computed.
template <class Path, class State>
__device__ __forceinline__ void tile_loop(const DecodeArgs& a, State& st, int seq, int kvh, int t0,
                                          int t1, int ctx, int lane) {
    constexpr int NL = Path::NL;
    const int tpb = a.tiles_per_block;
    const int32_t* bt = a.block_tables + static_cast<size_t>(seq) * a.max_blocks;
    int e_lo = t0 / tpb;
    const int e_last = (t1 - 1) / tpb;
    int win = load_window(bt, e_lo, e_last, lane, a.num_blocks);
    const u32x4* kc = static_cast<const u32x4*>(a.k_cache) + lane;
    const u32x4* vc = static_cast<const u32x4*>(a.v_cache) + lane;
    const size_t hkv = static_cast<size_t>(a.num_kv_heads);

    auto tile_off = [&](int t) -> size_t {
        const int e = t / tpb;
        if (e - e_lo >= kWave) {
            e_lo = e;
            win = load_window(bt, e_lo, e_last, lane, a.num_blocks);
        }
        const int blk = __builtin_amdgcn_readlane(win, e - e_lo);
        return ((static_cast<size_t>(blk) * hkv + kvh) * tpb + (t - e * tpb)) *
               static_cast<size_t>(Path::TILE_U4);
    };

    u32x4 kA[NL], vA[NL], kB[NL], vB[NL];
    size_t off = tile_off(t0);
#pragma unroll
    for (int s = 0; s < NL; ++s) kA[s] = kc[off + s * kWave];
#pragma unroll
    for (int s = 0; s < NL; ++s) vA[s] = vc[off + s * kWave];
    for (int t = t0; t < t1; t += 2) {
        if (t + 1 < t1) {
            off = tile_off(t + 1);
#pragma unroll
            for (int s = 0; s < NL; ++s) kB[s] = kc[off + s * kWave];
#pragma unroll
            for (int s = 0; s < NL; ++s) vB[s] = vc[off + s * kWave];
        }
        Path::tile(a, st, kA, vA, t, ctx, lane);
        if (t + 1 >= t1) break;
        if (t + 2 < t1) {
            off = tile_off(t + 2);
#pragma unroll
            for (int s = 0; s < NL; ++s) kA[s] = kc[off + s * kWave];
#pragma unroll
            for (int s = 0; s < NL; ++s) vA[s] = vc[off + s * kWave];
        }
        Path::tile(a, st, kB, vB, t + 1, ctx, lane);
    }
}

template <typename T, int D>
__device__ void HeadPath<T, D>::run_tiles(const DecodeArgs& a, State& st, int seq, int kvh, int t0,
                                          int t1, int ctx, int lane) {
    tile_loop<HeadPath<T, D>, State>(a, st, seq, kvh, t0, t1, ctx, lane);
}

template <int D>
__device__ void GroupPath<D>::run_tiles(const DecodeArgs& a, State& st, int seq, int kvh, int t0,
                                        int t1, int ctx, int lane) {
    tile_loop<GroupPath<D>, State>(a, st, seq, kvh, t0, t1, ctx, lane);
}

// ---------------------------------------------------------------------------------
// Pass 1: one wavefront per unit.
template <class Path, typename T, int D>
__global__ __launch_bounds__(64) void decode_pass1(DecodeArgs a) {
    const int lane = threadIdx.x;
    const int u = blockIdx.x;
    const int S = a.num_seqs;
    const int W = a.num_units;
    const size_t pf = static_cast<size_t>((a.heads_per_row * D + ((2 * a.heads_per_row + 3) & ~3)));
    // Sequences with no cached tokens get zeros; unit u covers sequences i == u (mod W).
    for (int i = u; i < S; i += W)
        if (ctx_of(a, i) == 0) write_zero_seq<T, D>(a, i, lane);
    // Tiles per row.
    int T_row = 0;
    for (int base = 0; base < S; base += kWave) {
        const int i = base + lane;
        T_row += wave_sum(i < S ? tiles_of(ctx_of(a, i)) : 0);
    }
    T_row = uni(T_row);
    int32_t* rec = a.unit_rec + static_cast<size_t>(u) * kRecInts;
    if (lane == 0) rec[0] = -1;  // overwritten below when the unit holds work
    const int total = a.rows * T_row;
    const int C = (total + W - 1) / W;
    const int start = u * C;
    if (total == 0 || start >= total) return;
    const int end = min(start + C, total);
    int row = start / T_row;
    const int tin = start - row * T_row;
    // Find the sequence holding tile `tin` of the row.
    int seq = 0, t0 = 0;
    {
        int carry = 0;
        for (int base = 0; base < S; base += kWave) {
            const int i = base + lane;
            const int n = i < S ? tiles_of(ctx_of(a, i)) : 0;
            const int incl = wave_inclusive_scan(n, lane) + carry;
            const unsigned long long hit = __ballot(incl > tin);
            if (hit) {
                const int f = __ffsll(static_cast<long long>(hit)) - 1;
                seq = base + f;
                t0 = tin - __shfl(incl - n, f);
                break;
            }
            carry = __shfl(incl, kWave - 1);
        }
    }
    seq = uni(seq);
    t0 = uni(t0);
    int pos = start;
    bool first = true;
    while (true) {
        const int nts = tiles_of(ctx_of(a, seq));
        const int take = min(nts - t0, end - pos);
        // Only reachable if context_lens changed under the kernel: stop rather than spin.
        if (take <= 0) break;
        const int seq_begin = pos - t0;
        if (first && lane == 0) {
            rec[0] = row;
            rec[1] = seq;
            rec[2] = seq_begin;
            rec[3] = seq_begin + nts;
            rec[4] = C;
        }
        const bool whole = (t0 == 0 && take == nts);
        float* prec = a.pieces + (static_cast<size_t>(u) * 2 + (first ? 0 : 1)) * pf;
        Path::piece(a, row, seq, t0, t0 + take, whole, prec, lane);
        pos += take;
        first = false;
        if (pos >= end) break;
        t0 = 0;
        do {
            if (++seq == S) {
                seq = 0;
                ++row;
            }
        } while (row < a.rows && tiles_of(ctx_of(a, seq)) == 0);
        if (row >= a.rows) break;
    }
}

// ---------------------------------------------------------------------------------
// Pass 2: unit u merges the split sequence whose last piece it holds (its first
// piece, when that sequence began in an earlier unit and ends inside unit u).
//   M = max_p m_p;  out = sum_p 2^(m_p - M) acc_p / sum_p 2^(m_p - M) l_p
template <typename T, int D>
__global__ __launch_bounds__(64) void decode_pass2(DecodeArgs a) {
    const int lane = threadIdx.x;
    const int u = blockIdx.x;
    const int32_t* rec = a.unit_rec + static_cast<size_t>(u) * kRecInts;
    const int row = rec[0];
    if (row < 0) return;
    const int seq = rec[1], begin = rec[2], end = rec[3], C = rec[4];
    if (seq < 0 || seq >= a.num_seqs || row >= a.rows || C <= 0 || begin < 0) return;
    const int ustart = u * C;
    if (begin >= ustart || end > ustart + C) return;
    const int us = begin / C;
    const int slot_us = (begin == us * C) ? 0 : 1;
    const int GH = a.heads_per_row;
    const size_t pf = static_cast<size_t>(GH * D + ((2 * GH + 3) & ~3));
    const int qh0 = row * GH;  // group rows hold heads row*G..; per-head rows hold head `row`
    T* o = static_cast<T*>(a.out) + (static_cast<size_t>(seq) * a.num_q_heads + qh0) * D;
    for (int idx = lane; idx < GH * D; idx += kWave) {
        const int h = idx / D;
        float M = kNegInf;
        for (int p = us; p <= u; ++p) {
            const float* r = a.pieces + (static_cast<size_t>(p) * 2 + (p == us ? slot_us : 0)) * pf;
            M = fmaxf(M, r[GH * D + h]);
        }
        float num = 0.f, den = 0.f;
        for (int p = us; p <= u; ++p) {
            const float* r = a.pieces + (static_cast<size_t>(p) * 2 + (p == us ? slot_us : 0)) * pf;
            const float w = fast_exp2(r[GH * D + h] - M);
            num = __builtin_fmaf(w, r[idx], num);
            den = __builtin_fmaf(w, r[GH * D + GH + h], den);
        }
        store_out<T>(o + idx, num / den);
    }
}

template <class Path, typename T, int D>
hipError_t launch_two_pass(const DecodeArgs& a, int passes, hipStream_t st) {
    if (passes & 1) {
        hipLaunchKernelGGL((decode_pass1<Path, T, D>), dim3(a.num_units), dim3(kWave), 0, st, a);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (passes & 2) {
        hipLaunchKernelGGL((decode_pass2<T, D>), dim3(a.num_units), dim3(kWave), 0, st, a);
        return hipGetLastError();
    }
    return hipSuccess;
}

}  // namespace

hipError_t launch_decode(int dtype, int head_dim, bool use_group_kernel, const DecodeArgs& a,
                         int passes, hipStream_t stream) {
    if (dtype == 1) {  // bf16
        if (use_group_kernel) {
            if (head_dim == 128) return launch_two_pass<GroupPath<128>, uint16_t, 128>(a, passes, stream);
            if (head_dim == 64) return launch_two_pass<GroupPath<64>, uint16_t, 64>(a, passes, stream);
        } else {
            if (head_dim == 128) return launch_two_pass<HeadPath<uint16_t, 128>, uint16_t, 128>(a, passes, stream);
            if (head_dim == 64) return launch_two_pass<HeadPath<uint16_t, 64>, uint16_t, 64>(a, passes, stream);
        }
    } else if (dtype == 0 && !use_group_kernel) {
        if (head_dim == 128) return launch_two_pass<HeadPath<uint32_t, 128>, uint32_t, 128>(a, passes, stream);
        if (head_dim == 64) return launch_two_pass<HeadPath<uint32_t, 64>, uint32_t, 64>(a, passes, stream);
    }
    return hipErrorInvalidValue;
}

}  // namespace pkv
