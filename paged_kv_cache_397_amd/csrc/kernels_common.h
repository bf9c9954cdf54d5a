// Device helpers shared by the decode and prefill kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

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

// s_waitcnt vmcnt(0): wait until every vector-memory load of the wave has returned
// (expcnt and lgkmcnt fields left at their maxima, i.e. not waited on).
__device__ __forceinline__ void wait_all_loads() { __builtin_amdgcn_s_waitcnt(0x0F70); }

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

template <typename T>
__device__ __forceinline__ void store_out(T* p, float x);
template <>
__device__ __forceinline__ void store_out<uint16_t>(uint16_t* p, float x) { *p = bf16_rne(x); }
template <>
__device__ __forceinline__ void store_out<uint32_t>(uint32_t* p, float x) {
    *p = __float_as_uint(x);
}

// ---------------------------------------------------------------------------------
// One 16-token tile folded into a group accumulator with the matrix cores.
//
// Sixteen columns share the K/V tile of one KV head: the G query heads of that
// head (decode, repeated with period G) or (query token, head) rows of a prompt
// chunk (prefill).  Lane l = 16 j + i owns column i.
//   S^T = K Q^T: v_mfma_f32_16x16x32_bf16, one per 32 dims; A = the K tile as
//     loaded (token i, dims 32 s + 8 j ..), B = the column's query (same dims).
//     Lane (j, i) gets the scores of tokens 4 j .. 4 j + 3 for column i.
//   Online softmax per column in base 2 (scores times scale * log2 e); P is
//     rounded to bf16 in the accumulator layout, which is the B operand of
//   O^T = V^T P^T: v_mfma_f32_16x16x16_bf16, one per 16 dims, fp32 accumulate.
//     acc[g][r] is dim 16 g + 4 j + r of column i.
// Token k of tile t is visible to lane's column when 16 t + k < lim (lim may differ
// per lane: the causal limit of a prefill row).  Value rows of tokens at or past
// vlim (the sequence length) are zeroed first: their slots may hold anything, and
// a zero weight times a NaN would still poison the sum; vlim must be uniform over
// the wave.  Every column must see at least one token of the first tile it folds, so
// that its running max is finite.
template <int D>
struct GroupAcc {
    float m, l;
    f32x4 acc[D / 16];
};

// kLazy: skip the accumulator rescale when no factor changed and mask V only on the
// sequence's last tile (bit-identical results).  It saves VALU work where the tile
// math bounds the kernel (prefill); the decode loop, bound by HBM, keeps the
// straight-line form, which needs fewer registers there.
template <int D, bool kLazy>
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
    if constexpr (!kLazy) {
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
        return;
    }
    // The accumulators sit in the matrix cores' registers, so a rescale costs a read,
    // a multiply and a write per element.  Once the running maxima settle, most tiles
    // leave every factor at exactly 1 (2^0), and multiplying by 1 changes no bit:
    // skip the rescale then.
    if (__ballot(alpha != 1.f)) {
#pragma unroll
        for (int g = 0; g < NG; ++g) st.acc[g] *= alpha;
    }
    auto pv = [&](uint32_t mask01, uint32_t mask23) {
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
    };
    if (t * kTile + kTile > vlim) {  // the sequence's last tile (vlim is uniform)
        const int nv = vlim - tok0;
        pv((nv > 0 ? 0x0000ffffu : 0u) | (nv > 1 ? 0xffff0000u : 0u),
           (nv > 2 ? 0x0000ffffu : 0u) | (nv > 3 ? 0xffff0000u : 0u));
    } else {
        pv(0xffffffffu, 0xffffffffu);
    }
}

}  // namespace
}  // namespace pkv
