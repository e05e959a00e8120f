// Decode attention when every query head has its own kv head (q_heads ==
// kv_heads), keys on the channel axis and values on the token axis: the
// decode step is a matrix-vector product per head, so it stays on the VALU
// and the kernel is organised around HBM streaming.
//
// Sources, by page title and section:
//   [N] nalar.dev, "Kuantisasi KV cache untuk mengurangi memory inferensi
//       long-context", "Kuantisasi dapat memindahkan pekerjaan ke decode path"
//       (unpack and apply scales inside the attention kernel)
//   [U] unite.ai (pt), "O Seu Cache KV Nao Tem um Problema de Bits...",
//       "Por Que o Cache KV E Onde Isso Morde" (decode reads the whole cache
//       once per generated token)
//
// Work decomposition: workgroup = (split of the token axis, kv head, seq);
// its 4 waves take interleaved 64-token super-tiles and never synchronise
// until the end. In a super-tile a lane owns one 32-channel unit (cg) of one
// token per sub-tile, so a wave reads whole rows with consecutive lanes on
// consecutive words.
//
// Keys: score_t = sum_u [ q.z_b over unit u ] + sum_c (q_c s_bc) code_tc. The
// per-block vector q_c s_bc and the per-unit sums of q_c z_bc are built once
// per block by the wave in LDS. Values: o_c = sum_t (p_t s_tg) code_tc +
// sum_t p_t z_tg.
//
// Code application: a masked uint32 holds two codes in its fp16 halves as
// integers code * 2^sh with sh + B <= 10, i.e. as fp16 subnormals of value
// code * 2^(sh-24); v_fma_mix_f32 multiplies such a half by an fp32 operand
// exactly, so one AND yields two products. The 2^(24-sh) factors are folded
// into the key vector; on the value side the softmax weights carry 2^24 (the
// reference maximum is lowered by 24) and the code shifts are undone at the end.
//
// Keys cached before the rotary embedding ([U] "Embebedos Rotatorios
// Complicam as Chaves": rotate after dequantization). The rotary
// instantiations (KVQ_MHA_ROPE, objects of their own) give a lane 16 whole
// channel pairs (i, i + D/2) of its token instead of a 32-channel unit: run A =
// channels 16cg..16cg+15, run B = their partners. With the query rotated to
// the position t0 of a 32-token half, Q = R(-t0) q, the score of the token at
// t0 + u is sum_i C_ui (Q_a k_a + Q_b k_b) + S_ui (Q_b k_a - Q_a k_b), where
// (C, S)_ui = (cos, sin)(u theta_i) comes from a table of the cache. With
// k = z + s code, each pair's two sums take four products of its two codes
// with weights built once per half and pair, so a code costs 3 VALU (1 on the
// plain path).
//
// Softmax: online in the log2 domain with a lazily moved reference maximum
// (moved only when a score exceeds it by more than 2^8), so rescaling is
// rare. Splits of one (seq, head) are merged by merge_kernel; a sequence that
// fits one split is written directly.
#include "kvq_append.h"
#include "kvq_device.h"
#include "kvq_internal.h"

#ifndef KVQ_MHA_ROPE
#define KVQ_MHA_ROPE 0
#endif

namespace kvq {
namespace {

using namespace dev;

__device__ __forceinline__ float mix_lo(uint32_t m, float b, float c) {
    float d;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(m), "v"(b), "v"(c));
    return d;
}
__device__ __forceinline__ float mix_hi(uint32_t m, float b, float c) {
    float d;
    asm("v_fma_mix_f32 %0, %1, %2, %3 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(m), "v"(b), "v"(c));
    return d;
}

// Bit position (within its fp16 half) at which channel j of a unit is applied.
template <int B>
__host__ __device__ constexpr int code_shift(int j) {
    if (B == 2) {
        const int r = j & 15;
        return r < 5 ? 2 * r : r < 8 ? 2 * (r - 5) : r < 13 ? 2 * (r - 8) : 2 * (r - 13);
    }
    if (B == 4) {
        const int r = j & 7;
        return r < 2 ? 4 * r : r < 4 ? 4 * (r - 2) : r < 6 ? 4 * (r - 4) : 4 * (r - 6);
    }
    return 0;
}

// Visit the 32 codes of one unit: f.pair<JL, JH>(m) gets a word whose low half
// holds code_JL << code_shift(JL) and high half code_JH << code_shift(JH);
// f.one<J>(c) gets code_J in the low half.
template <int B>
struct Unit;

template <>
struct Unit<2> {
    template <int Q, class F>
    static __device__ __forceinline__ void word(uint32_t x, F& f) {
        constexpr int J = 16 * Q;
        f.template pair<J + 0, J + 8>(x & 0x00030003u);
        f.template pair<J + 1, J + 9>(x & 0x000c000cu);
        f.template pair<J + 2, J + 10>(x & 0x00300030u);
        f.template pair<J + 3, J + 11>(x & 0x00c000c0u);
        f.template pair<J + 4, J + 12>(x & 0x03000300u);
        const uint32_t y = x >> 10;
        f.template pair<J + 5, J + 13>(y & 0x00030003u);
        f.template pair<J + 6, J + 14>(y & 0x000c000cu);
        f.template pair<J + 7, J + 15>(y & 0x00300030u);
    }
    template <class F>
    static __device__ __forceinline__ void visit(const uint32_t* w, F& f) {
        word<0>(w[0], f);
        word<1>(w[1], f);
    }
    template <int Q, class F>
    static __device__ __forceinline__ void word2(uint32_t x, uint32_t u, F& f) {
        constexpr int J = 16 * Q;
        f.template pair2<J + 0, J + 8>(x & 0x00030003u, u & 0x00030003u);
        f.template pair2<J + 1, J + 9>(x & 0x000c000cu, u & 0x000c000cu);
        f.template pair2<J + 2, J + 10>(x & 0x00300030u, u & 0x00300030u);
        f.template pair2<J + 3, J + 11>(x & 0x00c000c0u, u & 0x00c000c0u);
        f.template pair2<J + 4, J + 12>(x & 0x03000300u, u & 0x03000300u);
        const uint32_t y = x >> 10, v = u >> 10;
        f.template pair2<J + 5, J + 13>(y & 0x00030003u, v & 0x00030003u);
        f.template pair2<J + 6, J + 14>(y & 0x000c000cu, v & 0x000c000cu);
        f.template pair2<J + 7, J + 15>(y & 0x00300030u, v & 0x00300030u);
    }
    template <class F>
    static __device__ __forceinline__ void visit2(const uint32_t* w, const uint32_t* w2, F& f) {
        word2<0>(w[0], w2[0], f);
        word2<1>(w[1], w2[1], f);
    }
};

template <>
struct Unit<4> {
    template <int Q, class F>
    static __device__ __forceinline__ void word(uint32_t x, F& f) {
        constexpr int J = 8 * Q;
        f.template pair<J + 0, J + 4>(x & 0x000f000fu);
        f.template pair<J + 1, J + 5>(x & 0x00f000f0u);
        const uint32_t y = x >> 8;
        f.template pair<J + 2, J + 6>(y & 0x000f000fu);
        f.template pair<J + 3, J + 7>(y & 0x00f000f0u);
    }
    template <class F>
    static __device__ __forceinline__ void visit(const uint32_t* w, F& f) {
        word<0>(w[0], f);
        word<1>(w[1], f);
        word<2>(w[2], f);
        word<3>(w[3], f);
    }
    template <int Q, class F>
    static __device__ __forceinline__ void word2(uint32_t x, uint32_t u, F& f) {
        constexpr int J = 8 * Q;
        f.template pair2<J + 0, J + 4>(x & 0x000f000fu, u & 0x000f000fu);
        f.template pair2<J + 1, J + 5>(x & 0x00f000f0u, u & 0x00f000f0u);
        const uint32_t y = x >> 8, v = u >> 8;
        f.template pair2<J + 2, J + 6>(y & 0x000f000fu, v & 0x000f000fu);
        f.template pair2<J + 3, J + 7>(y & 0x00f000f0u, v & 0x00f000f0u);
    }
    template <class F>
    static __device__ __forceinline__ void visit2(const uint32_t* w, const uint32_t* w2, F& f) {
        word2<0>(w[0], w2[0], f);
        word2<1>(w[1], w2[1], f);
        word2<2>(w[2], w2[2], f);
        word2<3>(w[3], w2[3], f);
    }
};

template <>
struct Unit<8> {
    template <int Q, class F>
    static __device__ __forceinline__ void word(uint32_t x, F& f) {
        constexpr int J = 4 * Q;
        f.template pair<J + 0, J + 2>(x & 0x00ff00ffu);
        f.template pair<J + 1, J + 3>(__builtin_amdgcn_perm(x, x, 0x0c070c05u));
    }
    template <class F>
    static __device__ __forceinline__ void visit(const uint32_t* w, F& f) {
        word<0>(w[0], f);
        word<1>(w[1], f);
        word<2>(w[2], f);
        word<3>(w[3], f);
        word<4>(w[4], f);
        word<5>(w[5], f);
        word<6>(w[6], f);
        word<7>(w[7], f);
    }
    template <int Q, class F>
    static __device__ __forceinline__ void word2(uint32_t x, uint32_t u, F& f) {
        constexpr int J = 4 * Q;
        f.template pair2<J + 0, J + 2>(x & 0x00ff00ffu, u & 0x00ff00ffu);
        f.template pair2<J + 1, J + 3>(__builtin_amdgcn_perm(x, x, 0x0c070c05u), __builtin_amdgcn_perm(u, u, 0x0c070c05u));
    }
    template <class F>
    static __device__ __forceinline__ void visit2(const uint32_t* w, const uint32_t* w2, F& f) {
        word2<0>(w[0], w2[0], f);
        word2<1>(w[1], w2[1], f);
        word2<2>(w[2], w2[2], f);
        word2<3>(w[3], w2[3], f);
        word2<4>(w[4], w2[4], f);
        word2<5>(w[5], w2[5], f);
        word2<6>(w[6], w2[6], f);
        word2<7>(w[7], w2[7], f);
    }
};

// 3- and 6-bit codes straddle words: one bit-field extract per code.
template <int B>
struct UnitStraddle {
    template <int J, class F>
    static __device__ __forceinline__ void one(const uint32_t* w, F& f) {
        constexpr int pos = J * B, wi = pos >> 5, sh = pos & 31;
        uint32_t c;
        if constexpr (sh + B <= 32) {
            c = (w[wi] >> sh) & ((1u << B) - 1u);
        } else {
            c = __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << B) - 1u);
        }
        f.template one<J>(c);
    }
    template <int J, class F>
    static __device__ __forceinline__ void rec(const uint32_t* w, F& f) {
        if constexpr (J < 32) {
            one<J>(w, f);
            rec<J + 1>(w, f);
        }
    }
    template <class F>
    static __device__ __forceinline__ void visit(const uint32_t* w, F& f) {
        rec<0>(w, f);
    }
    template <int J>
    static __device__ __forceinline__ uint32_t code(const uint32_t* w) {
        constexpr int pos = J * B, wi = pos >> 5, sh = pos & 31;
        if constexpr (sh + B <= 32) return (w[wi] >> sh) & ((1u << B) - 1u);
        else return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << B) - 1u);
    }
    template <int J, class F>
    static __device__ __forceinline__ void rec2(const uint32_t* w, const uint32_t* w2, F& f) {
        if constexpr (J < 32) {
            f.template one2<J>(code<J>(w), code<J>(w2));
            rec2<J + 1>(w, w2, f);
        }
    }
    template <class F>
    static __device__ __forceinline__ void visit2(const uint32_t* w, const uint32_t* w2, F& f) {
        rec2<0>(w, w2, f);
    }
};
template <>
struct Unit<3> : UnitStraddle<3> {};
template <>
struct Unit<6> : UnitStraddle<6> {};

// Dot product of one unit's codes with 32 prescaled key weights.
struct KeyDot {
    const float* qv;
    float a0, a1;
    template <int JL, int JH>
    __device__ __forceinline__ void pair(uint32_t m) {
        a0 = mix_lo(m, qv[JL], a0);
        a1 = mix_hi(m, qv[JH], a1);
    }
    template <int J>
    __device__ __forceinline__ void one(uint32_t c) {
        if constexpr (J & 1) a1 = mix_lo(c, qv[J], a1);
        else a0 = mix_lo(c, qv[J], a0);
    }
};

// Two tokens at once: four independent accumulation chains.
struct KeyDot2 {
    const float* qv;
    float a0, a1, b0, b1;
    template <int JL, int JH>
    __device__ __forceinline__ void pair2(uint32_t m, uint32_t n) {
        a0 = mix_lo(m, qv[JL], a0);
        b0 = mix_lo(n, qv[JL], b0);
        a1 = mix_hi(m, qv[JH], a1);
        b1 = mix_hi(n, qv[JH], b1);
    }
    template <int J>
    __device__ __forceinline__ void one2(uint32_t c, uint32_t d) {
        if constexpr (J & 1) {
            a1 = mix_lo(c, qv[J], a1);
            b1 = mix_lo(d, qv[J], b1);
        } else {
            a0 = mix_lo(c, qv[J], a0);
            b0 = mix_lo(d, qv[J], b0);
        }
    }
};

// Rotary layout: the words of a 16-code run (a run of 3-bit codes starts on
// a half word when cg is odd: two words, aligned at use).
template <int B>
__host__ __device__ constexpr int run_words() { return B == 3 ? 2 : B / 2; }

// Visit the 16 code pairs of runs A and B (same token): f.pair2<JL, JH>(mA, mB)
// gets run A's and run B's words masked to codes JL (low half) and JH (high
// half), each at bit code_shift(J) of its half; f.one2<J>(cA, cB) the codes
// themselves. `sh` is the run's bit offset in its first word (0, or 16 for
// 3-bit runs of odd cg).
template <int B, class F>
__device__ __forceinline__ void visit_runs(const uint32_t* w, int sh, F& f) {
    constexpr int RW = run_words<B>();
    if constexpr (B == 2) {
        Unit<2>::word2<0>(w[0], w[RW], f);
    } else if constexpr (B == 4) {
        Unit<4>::word2<0>(w[0], w[RW], f);
        Unit<4>::word2<1>(w[1], w[RW + 1], f);
    } else if constexpr (B == 8) {
        static_for<4>([&](auto Q) { Unit<8>::word2<Q>(w[Q], w[RW + Q], f); });
    } else {
        uint32_t a[RW], b[RW];
        if constexpr (B == 3) {
            a[0] = __builtin_amdgcn_alignbit(w[1], w[0], sh);
            a[1] = w[1] >> sh;
            b[0] = __builtin_amdgcn_alignbit(w[3], w[2], sh);
            b[1] = w[3] >> sh;
        } else {
#pragma unroll
            for (int k = 0; k < RW; ++k) a[k] = w[k], b[k] = w[RW + k];
        }
        static_for<16>([&](auto J) {
            constexpr int j = J;
            f.template one2<j>(UnitStraddle<B>::template code<j>(a), UnitStraddle<B>::template code<j>(b));
        });
    }
}

// LDS layout of the rotary (cos, sin) table: pair-major, [pair][u] as float
// pairs, 68 floats per pair (33 offsets and 2 spare), a group of 16 pairs 16
// floats after the previous one. The 16 lanes of a quarter wave (4 offsets x
// 4 pair groups) then read 8-byte words on 16 distinct bank pairs.
constexpr int kRopePairStride = 68;
__host__ __device__ constexpr int rope_lds_off(int pair, int u) { return kRopePairStride * pair + 8 * (pair >> 4) + 2 * u; }

// The same for two tokens of one 32-token half (w0, w1), which share the
// pair weights: f.pair4<JL, JH>(mA0, mB0, mA1, mB1), f.one4<J>(cA0, cB0, cA1, cB1).
template <int JL, int JH, class F>
__device__ __forceinline__ void mask4(F& f, uint32_t a0, uint32_t b0, uint32_t a1, uint32_t b1, uint32_t m) {
    f.template pair4<JL, JH>(a0 & m, b0 & m, a1 & m, b1 & m);
}
template <int B, class F>
__device__ __forceinline__ void visit_runs2(const uint32_t* w0, const uint32_t* w1, int sh, F& f) {
    constexpr int RW = run_words<B>();
    if constexpr (B == 2) {  // the masks of Unit<2>::word
        const uint32_t a0 = w0[0], b0 = w0[RW], a1 = w1[0], b1 = w1[RW];
        mask4<0, 8>(f, a0, b0, a1, b1, 0x00030003u);
        mask4<1, 9>(f, a0, b0, a1, b1, 0x000c000cu);
        mask4<2, 10>(f, a0, b0, a1, b1, 0x00300030u);
        mask4<3, 11>(f, a0, b0, a1, b1, 0x00c000c0u);
        mask4<4, 12>(f, a0, b0, a1, b1, 0x03000300u);
        const uint32_t c0 = a0 >> 10, d0 = b0 >> 10, c1 = a1 >> 10, d1 = b1 >> 10;
        mask4<5, 13>(f, c0, d0, c1, d1, 0x00030003u);
        mask4<6, 14>(f, c0, d0, c1, d1, 0x000c000cu);
        mask4<7, 15>(f, c0, d0, c1, d1, 0x00300030u);
    } else if constexpr (B == 4) {  // Unit<4>::word
        static_for<2>([&](auto Q) {
            constexpr int J = 8 * Q;
            const uint32_t a0 = w0[Q], b0 = w0[RW + Q], a1 = w1[Q], b1 = w1[RW + Q];
            mask4<J + 0, J + 4>(f, a0, b0, a1, b1, 0x000f000fu);
            mask4<J + 1, J + 5>(f, a0, b0, a1, b1, 0x00f000f0u);
            mask4<J + 2, J + 6>(f, a0 >> 8, b0 >> 8, a1 >> 8, b1 >> 8, 0x000f000fu);
            mask4<J + 3, J + 7>(f, a0 >> 8, b0 >> 8, a1 >> 8, b1 >> 8, 0x00f000f0u);
        });
    } else if constexpr (B == 8) {  // Unit<8>::word
        static_for<4>([&](auto Q) {
            constexpr int J = 4 * Q;
            const uint32_t a0 = w0[Q], b0 = w0[RW + Q], a1 = w1[Q], b1 = w1[RW + Q];
            mask4<J + 0, J + 2>(f, a0, b0, a1, b1, 0x00ff00ffu);
            f.template pair4<J + 1, J + 3>(
                __builtin_amdgcn_perm(a0, a0, 0x0c070c05u), __builtin_amdgcn_perm(b0, b0, 0x0c070c05u),
                __builtin_amdgcn_perm(a1, a1, 0x0c070c05u), __builtin_amdgcn_perm(b1, b1, 0x0c070c05u));
        });
    } else {
        uint32_t a[2][RW], b[2][RW];
#pragma unroll
        for (int t = 0; t < 2; ++t) {
            const uint32_t* w = t ? w1 : w0;
            if constexpr (B == 3) {
                a[t][0] = __builtin_amdgcn_alignbit(w[1], w[0], sh);
                a[t][1] = w[1] >> sh;
                b[t][0] = __builtin_amdgcn_alignbit(w[3], w[2], sh);
                b[t][1] = w[3] >> sh;
            } else {
#pragma unroll
                for (int k = 0; k < RW; ++k) a[t][k] = w[k], b[t][k] = w[RW + k];
            }
        }
        static_for<16>([&](auto J) {
            constexpr int j = J;
            f.template one4<j>(UnitStraddle<B>::template code<j>(a[0]), UnitStraddle<B>::template code<j>(b[0]),
                               UnitStraddle<B>::template code<j>(a[1]), UnitStraddle<B>::template code<j>(b[1]));
        });
    }
}

// Rotary score of one token over the lane's 16 pairs J: w4[J] = {Q_a s_a,
// Q_b s_b, Q_a z_a + Q_b z_b, Q_b s_a}, w2[J] = {-Q_a s_b, Q_b z_a - Q_a z_b}
// (steps with the 2^(24 - code_shift(J)) factor of the code halves), cs[kRopePairStride J] =
// (C, S) of the token's offset: a0 = sum C A, a1 = sum S B.
struct RopeDot {
    const float4* w4;
    const float2* w2;
    const float* cs;
    float a0, a1;
    template <int J, bool HI>
    __device__ __forceinline__ void pair_j(uint32_t mA, uint32_t mB) {
        const float4 w = w4[J];
        const float2 v = w2[J];
        const float2 c = *(const float2*)&cs[kRopePairStride * J];
        float A, Bs;
        if constexpr (HI) {
            A = mix_hi(mB, w.y, mix_hi(mA, w.x, w.z));
            Bs = mix_hi(mB, v.x, mix_hi(mA, w.w, v.y));
        } else {
            A = mix_lo(mB, w.y, mix_lo(mA, w.x, w.z));
            Bs = mix_lo(mB, v.x, mix_lo(mA, w.w, v.y));
        }
        a0 = fmaf(c.x, A, a0);
        a1 = fmaf(c.y, Bs, a1);
    }
    template <int JL, int JH>
    __device__ __forceinline__ void pair2(uint32_t mA, uint32_t mB) {
        pair_j<JL, false>(mA, mB);
        pair_j<JH, true>(mA, mB);
    }
    template <int J>
    __device__ __forceinline__ void one2(uint32_t cA, uint32_t cB) {
        pair_j<J, false>(cA, cB);
    }
};

// Two tokens of one half (offsets cs0, cs1), one load of the pair weights.
struct RopeDot2 {
    const float4* w4;
    const float2* w2;
    const float* cs0;
    const float* cs1;
    float a0, a1, b0, b1;  // token 0: sum C A, sum S B; token 1: the same
    template <int J, bool HI>
    __device__ __forceinline__ void pair_j(uint32_t mA0, uint32_t mB0, uint32_t mA1, uint32_t mB1) {
        const float4 w = w4[J];
        const float2 v = w2[J];
        const float2 c = *(const float2*)&cs0[kRopePairStride * J], d = *(const float2*)&cs1[kRopePairStride * J];
        float A0, B0, A1, B1;
        if constexpr (HI) {
            A0 = mix_hi(mB0, w.y, mix_hi(mA0, w.x, w.z));
            B0 = mix_hi(mB0, v.x, mix_hi(mA0, w.w, v.y));
            A1 = mix_hi(mB1, w.y, mix_hi(mA1, w.x, w.z));
            B1 = mix_hi(mB1, v.x, mix_hi(mA1, w.w, v.y));
        } else {
            A0 = mix_lo(mB0, w.y, mix_lo(mA0, w.x, w.z));
            B0 = mix_lo(mB0, v.x, mix_lo(mA0, w.w, v.y));
            A1 = mix_lo(mB1, w.y, mix_lo(mA1, w.x, w.z));
            B1 = mix_lo(mB1, v.x, mix_lo(mA1, w.w, v.y));
        }
        a0 = fmaf(c.x, A0, a0);
        a1 = fmaf(c.y, B0, a1);
        b0 = fmaf(d.x, A1, b0);
        b1 = fmaf(d.y, B1, b1);
    }
    template <int JL, int JH>
    __device__ __forceinline__ void pair4(uint32_t mA0, uint32_t mB0, uint32_t mA1, uint32_t mB1) {
        pair_j<JL, false>(mA0, mB0, mA1, mB1);
        pair_j<JH, true>(mA0, mB0, mA1, mB1);
    }
    template <int J>
    __device__ __forceinline__ void one4(uint32_t cA0, uint32_t cB0, uint32_t cA1, uint32_t cB1) {
        pair_j<J, false>(cA0, cB0, cA1, cB1);
    }
};

// Full-precision rotary score over the lane's 16 pairs: q4[J] = {Q_a, Q_b}
// of the token's anchor (x, y or z, w: `second`), rows xa (run A) and xb (run B).
__device__ __forceinline__ float rope_row_score(const float4* q4, bool second, const float* cs, const float (&xa)[16],
                                                const float (&xb)[16]) {
    float a0 = 0.f, a1 = 0.f;
#pragma unroll
    for (int j = 0; j < 16; ++j) {
        const float4 q = q4[j];
        const float qa = second ? q.z : q.x, qb = second ? q.w : q.y;
        const float2 c = *(const float2*)&cs[kRopePairStride * j];
        a0 = fmaf(c.x, fmaf(qa, xa[j], qb * xb[j]), a0);
        a1 = fmaf(c.y, fmaf(qb, xa[j], -(qa * xb[j])), a1);
    }
    return a0 + a1;
}

// acc[j] += w * code_j * 2^code_shift(j)  (w carries the 2^24 factor).
struct ValueAxpy {
    float w;
    float* acc;
    template <int JL, int JH>
    __device__ __forceinline__ void pair(uint32_t m) {
        acc[JL] = mix_lo(m, w, acc[JL]);
        acc[JH] = mix_hi(m, w, acc[JH]);
    }
    template <int J>
    __device__ __forceinline__ void one(uint32_t c) {
        acc[J] = mix_lo(c, w, acc[J]);
    }
};

template <int B>
__device__ __forceinline__ void load_words(const uint32_t* p, uint32_t* w) {
    if constexpr (B == 2) {
        const uint2 v = ld_stream2(p);
        w[0] = v.x;
        w[1] = v.y;
    } else if constexpr (B == 4) {
        const uint4 v = ld_stream4(p);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    } else if constexpr (B == 8) {
        const uint4 v0 = ld_stream4(p);
        const uint4 v1 = ld_stream4(p + 4);
        w[0] = v0.x;
        w[1] = v0.y;
        w[2] = v0.z;
        w[3] = v0.w;
        w[4] = v1.x;
        w[5] = v1.y;
        w[6] = v1.z;
        w[7] = v1.w;
    } else if constexpr (B == 6) {
        const uint2* q = (const uint2*)p;  // a 24-byte unit is 8-byte aligned
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            const uint2 v = ld_stream2((const uint32_t*)(q + k));
            w[2 * k] = v.x;
            w[2 * k + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int k = 0; k < B; ++k) w[k] = ld_stream(p + k);
    }
}

// The words of a 16-code run of the rotary layout, starting at word p.
template <int B>
__device__ __forceinline__ void load_run(const uint32_t* p, uint32_t* w) {
    if constexpr (B == 2) {
        w[0] = ld_stream(p);
    } else if constexpr (B == 4) {
        const uint2 v = ld_stream2(p);
        w[0] = v.x;
        w[1] = v.y;
    } else if constexpr (B == 8) {
        const uint4 v = ld_stream4(p);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    } else {  // 3 and 6 bits: runs start on any word
#pragma unroll
        for (int k = 0; k < run_words<B>(); ++k) w[k] = ld_stream(p + k);
    }
}

template <int CTRL>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Sum over the N consecutive lanes (N = 2, 4, 8) that hold the units of one token.
template <int N>
__device__ __forceinline__ float group_sum(float v) {
    v += dpp_f<0xb1>(v);  // quad_perm [1,0,3,2]
    if constexpr (N >= 4) v += dpp_f<0x4e>(v);  // quad_perm [2,3,0,1]
    if constexpr (N >= 8) v += dpp_f<0x141>(v);  // row_half_mirror
    return v;
}

__device__ __forceinline__ float wave_max_f(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

__device__ __forceinline__ void wave_sync_lds() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__device__ __forceinline__ float load_in_rt(const void* p, size_t i, int dt) {
    if (dt == 0) return load_in<0>(p, i);
    if (dt == 1) return load_in<1>(p, i);
    return load_in<2>(p, i);
}

__device__ __forceinline__ void load16_rt(const void* p, size_t off, int dt, float (&x)[16]) {
    if (dt == 0) load16<0>(p, off, x);
    else if (dt == 1) load16<1>(p, off, x);
    else load16<2>(p, off, x);
}

constexpr float kTwo24 = 16777216.0f;

constexpr float kRescale = 8.0f;  // log2-domain slack before the reference maximum moves

// Registers of one 64-token super-tile: the lane's key and value unit words,
// value metadata, and the key metadata of the super-tile's blocks.
// Rotary instantiations: runs A and B of the lane's 16 pairs per token, and
// the key metadata of channels p and p + D/2 of the lane's prologue pairs p.
template <int D, int BK, int BV, bool ROPE>
struct Stage {
    static constexpr int UPR = D / 32;
    static constexpr int KW = ROPE ? 2 * run_words<BK>() : BK;
    static constexpr int KM = ROPE ? 2 * (D >= 128 ? D / 128 : 1) : D / 64;
    uint32_t kw[UPR][KW];
    uint32_t vw[UPR][BV];
    uint32_t vmw[UPR];
    uint32_t kmw[2][KM];
};

template <int N>
__device__ __forceinline__ void load_words_n(const uint32_t* p, uint32_t* w) {
    if constexpr (N == 1) {
        w[0] = ld_stream(p);
    } else if constexpr (N == 2) {
        const uint2 v = ld_stream2(p);
        w[0] = v.x;
        w[1] = v.y;
    } else {
        const uint4 v = ld_stream4(p);
        w[0] = v.x;
        w[1] = v.y;
        w[2] = v.z;
        w[3] = v.w;
    }
}

template <int N>
__device__ __forceinline__ void store_lds_n(float* p, const float* v) {
    if constexpr (N == 1) {
        p[0] = v[0];
    } else if constexpr (N == 2) {
        *(float2*)p = make_float2(v[0], v[1]);
    } else {
        *(float4*)p = make_float4(v[0], v[1], v[2], v[3]);
    }
}

// Sum over aligned groups of N lanes (N = 8, 16 or 32).
template <int N>
__device__ __forceinline__ float unit_sum(float v) {
    v += dpp_f<0xb1>(v);
    v += dpp_f<0x4e>(v);
    v += dpp_f<0x141>(v);  // row_half_mirror: 8-lane sums
    if constexpr (N >= 16) v += dpp_f<0x140>(v);  // row_mirror: 16-lane sums
    if constexpr (N >= 32) v += __shfl_xor(v, 16);
    return v;
}

// Fused decode step: append the new rows of (seq, head), which only the
// last split's residual loop (or full-precision loop) reads: values quantized
// per row (one thread per 32-channel unit, rows of whole groups), keys copied
// into the residual, and with a window both copied into the window area.
__device__ __forceinline__ void fused_append(const DecodeArgs& a, int head, int seq, int len0, int n, int nthreads) {
    const int UPR = a.head_dim >> 5;
    const int r = (int)threadIdx.x / UPR, u = (int)threadIdx.x % UPR;
    if (a.in_dtype == 0) {
        if (r < n) token_axis_row<0>(a.app_v, r, u, head, seq, len0);
        residual_rows<0>(a.app_k, head, seq, len0, len0, len0 + n, nthreads);
        if (a.win_mode) window_rows<0>(a.app_k, a.app_v, seq, head, 0, 1, nthreads);
    } else if (a.in_dtype == 1) {
        if (r < n) token_axis_row<1>(a.app_v, r, u, head, seq, len0);
        residual_rows<1>(a.app_k, head, seq, len0, len0, len0 + n, nthreads);
        if (a.win_mode) window_rows<1>(a.app_k, a.app_v, seq, head, 0, 1, nthreads);
    } else {
        if (r < n) token_axis_row<2>(a.app_v, r, u, head, seq, len0);
        residual_rows<2>(a.app_k, head, seq, len0, len0, len0 + n, nthreads);
        if (a.win_mode) window_rows<2>(a.app_k, a.app_v, seq, head, 0, 1, nthreads);
    }
}

// FUSED: the instantiation of the fused decode step (the append prologue is
// compiled only there, so the attention loop of the plain call is unchanged).
// ROPE: keys cached before the rotary embedding.
// The rotary object keeps two waves per SIMD (the plain kernel fits there by itself).
#if KVQ_MHA_ROPE
#define KVQ_MHA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(2, 2)))
#else
#define KVQ_MHA_OCCUPANCY
#endif
template <int D, int BK, int BV, int NW, int NS, bool FUSED, bool ROPE>
__global__ __launch_bounds__(NW * 64) KVQ_MHA_OCCUPANCY void decode_mha_kernel(DecodeArgs a0) {
    int z = blockIdx.z;
    const DecodeArgs a = layer_args(a0, z, gridDim.z / a0.n_layers);
    constexpr int UPR = D / 32;   // units per row = lanes per token
    constexpr int TPW = 64 / UPR; // tokens per sub-tile
    constexpr int KPL = D / 64;   // channels per lane in the per-block prologue
    constexpr int HALF = UPR / 2; // sub-tiles per 32 tokens
    using St = Stage<D, BK, BV, ROPE>;

    __shared__ float q_lds[D];
    constexpr int QSP = 36;         // padded floats per unit row of the key vector (bank spread)
    __shared__ float qs_lds[NW][2][UPR * QSP];
    __shared__ float bz_lds[NW][2][UPR];
    __shared__ float mrg_o[NW][D];
    __shared__ float mrg_ml[NW][2];
    constexpr int NT = NW * 64;  // threads
    // Rotary keys: the (cos, sin) table of the cache (rope_lds_off layout);
    // per wave and 32-token half the weights of the D/2 pairs (slot
    // p + p / 16: a lane's 16 pairs are contiguous, groups one slot apart), or
    // in the full-precision loops the rotated query pairs of two anchors.
    constexpr int NPS = D / 2 + D / 32;
    constexpr int KPP = D >= 128 ? D / 128 : 1;  // prologue pairs per lane (p = lane + 64k < D/2)
    __shared__ __align__(16) float rt_lds[ROPE ? rope_lds_off(D / 2, 0) : 1];
    __shared__ float4 pw4_lds[ROPE ? NW : 1][2][ROPE ? NPS : 1];
    __shared__ float2 pw2_lds[ROPE ? NW : 1][2][ROPE ? NPS : 1];

    const int seq = a.seq_list ? a.seq_list[z] : z;
    const int kvh = blockIdx.y, split = blockIdx.x;
    const int len_old = a.len[seq];
    const int n_app = FUSED ? (a.app_v.n_new ? a.app_v.n_new[seq] : a.app_v.n_uniform) : 0;
    const int len = len_old + n_app;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    if (FUSED && kvh == 0 && split == 0 && tid == 0) a.app_k.len_out[seq] = len;
    float* out = a.out + ((size_t)seq * a.q_heads + kvh) * D;
    if (len == 0) {
        if (split == 0)
            for (int c = tid; c < D; c += NT) out[c] = 0.f;
        return;
    }
    // Quantized tokens [tb, te): all of them, or with a full-precision window
    // the whole key blocks inside [sinks, len - window), whose last split also
    // attends the full-precision rows (possibly with no quantized token).
    int tb, te;
    quant_range(a, len, tb, te);
    const int CW = a.chunk;
    const int nsplit = max(1, (te - tb) / CW);
    if (split >= nsplit) return;
    // Fused step: the new rows are only read by this split's residual loop, so
    // their stores complete while the quantized tokens stream; the barrier
    // before that loop (workgroup scope: one compute unit) orders them.
    const bool appended = FUSED && n_app > 0 && split == nsplit - 1;
    if (appended) fused_append(a, kvh, seq, len_old, n_app, NT);
    const int wa = tb + split * CW, wb = split == nsplit - 1 ? te : wa + CW;
    const int ts = lane / UPR, cg = lane % UPR;
    const SeqEntry& e = a.table[seq];
    const int lgk = a.log2_group_k;
    const bool two_blocks = lgk == 5;  // a 64-token super-tile spans two 32-token key blocks
    const int nqk = a.win_mode ? te : (len >> lgk) << lgk;
    const int qend = min(wb, nqk);

    // head kvh's codes and metadata inside a page (pool offsets with contiguous storage)
    const uint8_t* kc = a.codes + e.codes[0] + (size_t)kvh * e.codes_hs[0];
    const uint8_t* km = a.meta + e.meta[0] + (size_t)kvh * e.meta_hs[0];
    const uint8_t* kr = a.resid + e.resid[0] + (size_t)kvh * e.resid_hs[0];
    const uint8_t* vc = a.codes + e.codes[1] + (size_t)kvh * e.codes_hs[1];
    const uint8_t* vm = a.meta + e.meta[1] + (size_t)kvh * e.meta_hs[1];
    const int lgv = a.log2_group_v;
    const int vgpr = D >> lgv;           // value groups per row
    const int vg = (32 * cg) >> lgv;     // this lane's value group

    for (int c = tid; c < D; c += NT)
        q_lds[c] = load_in_rt(a.q, ((size_t)seq * a.q_heads + kvh) * D + c, a.in_dtype) * a.qscale;
    double th[KPP];  // rotary frequencies of the lane's prologue pairs
    if constexpr (ROPE) {
        for (int i = tid; i < kRopeRows * (D / 2); i += NT) {
            const int u = i / (D / 2), pp = i - u * (D / 2);
            *(float2*)&rt_lds[rope_lds_off(pp, u)] = ((const float2*)a.rope_tab)[i];
        }
#pragma unroll
        for (int k = 0; k < KPP; ++k) th[k] = a.rope_theta[min(lane + 64 * k, D / 2 - 1)];
    }
    __syncthreads();

    // per-lane constants of the per-block prologue: q_c and q_c * 2^(24 - shift(c))
    float qk[KPL], qks[KPL];
#pragma unroll
    for (int k = 0; k < KPL; ++k) {
        const int c = KPL * lane + k;
        qk[k] = q_lds[c];
        qks[k] = qk[k] * (float)(1 << (24 - code_shift<BK>(c & 31)));
    }

    float acc[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = 0.f;
    // Every weight carries a 2^24 factor (the reference is m - 24), which the
    // fp16-subnormal code products need; it cancels between o and l.
    float zacc = 0.f, lsum = 0.f, m = -INFINITY;

    // Issue every global load of the super-tile starting at st. The number of
    // loads never depends on st (addresses past the quantized range are clamped
    // into it and the data is ignored), so the compiler can count outstanding
    // loads exactly and keep the later stages in flight.
    const int tlast = qend - 1;
    const int blast = tlast >> lgk;
    // Pages: a super-tile (64-aligned, pages hold a multiple of 64 tokens) lies
    // in one page. Lane k of pev holds the page of this wave's k-th super-tile,
    // clamped like the loads (the host keeps a split within 64 of them), so the
    // loop reads it with a lane read instead of a dependent memory load.
    const int st0 = wa + 64 * wave;
    constexpr int STEP = NW * 64;
    const int psh = e.page_shift;
    // (contiguous storage, page stride 0, skips the load: the first loads do not wait for it)
    const bool paged = e.page_bytes != 0;
    uint32_t pev = 0;
    if (paged && st0 < qend) pev = a.pages[e.page_list + (min(st0 + STEP * lane, tlast) >> psh)];
    auto load_stage = [&](int st, St& r) {
        const int sc0 = min(st, tlast);
        const uint64_t pb =
            paged ? (uint64_t)(uint32_t)__builtin_amdgcn_readlane(pev, min((st - st0) / STEP, 63)) * e.page_bytes : 0;
        const int ps = (sc0 >> psh) << psh;  // first token of the page
        const int t0 = st + ts;
#pragma unroll
        for (int s = 0; s < UPR; ++s) {
            const int t = min(t0 + s * TPW, tlast) - ps;
            const uint32_t* krow = (const uint32_t*)(kc + pb + (size_t)t * (D * BK / 8));
            if constexpr (ROPE) {
                load_run<BK>(krow + ((16 * BK * cg) >> 5), r.kw[s]);
                load_run<BK>(krow + ((16 * BK * cg) >> 5) + D * BK / 64, r.kw[s] + run_words<BK>());
            } else {
                load_words<BK>(krow + cg * BK, r.kw[s]);
            }
            load_words<BV>((const uint32_t*)(vc + pb + (size_t)t * (D * BV / 8)) + cg * BV, r.vw[s]);
            r.vmw[s] = ld_stream((const uint32_t*)(vm + pb) + (size_t)t * vgpr + vg);
        }
        const int b0 = sc0 >> lgk;
        const int b1 = (two_blocks ? min(b0 + 1, blast) : b0) - (ps >> lgk);
        const uint32_t* kmp = (const uint32_t*)(km + pb);
        if constexpr (ROPE) {
#pragma unroll
            for (int k = 0; k < KPP; ++k) {
                const int pp = min(lane + 64 * k, D / 2 - 1);
                r.kmw[0][2 * k] = ld_stream(kmp + (size_t)(b0 - (ps >> lgk)) * D + pp);
                r.kmw[0][2 * k + 1] = ld_stream(kmp + (size_t)(b0 - (ps >> lgk)) * D + pp + D / 2);
                r.kmw[1][2 * k] = ld_stream(kmp + (size_t)b1 * D + pp);
                r.kmw[1][2 * k + 1] = ld_stream(kmp + (size_t)b1 * D + pp + D / 2);
            }
        } else {
            load_words_n<KPL>(kmp + (size_t)(b0 - (ps >> lgk)) * D + KPL * lane, r.kmw[0]);
            load_words_n<KPL>(kmp + (size_t)b1 * D + KPL * lane, r.kmw[1]);
        }
    };

    // Online softmax over this lane's UPR scores (one per sub-tile), then the value rows.
    auto softmax_and_values = [&](const float (&sc)[UPR], const uint32_t (&vw)[UPR][BV], const uint32_t (&vmw)[UPR],
                                  const bool (&valid)[UPR]) {
        float tmax = sc[0];
#pragma unroll
        for (int s = 1; s < UPR; ++s) tmax = fmaxf(tmax, sc[s]);
        if (m == -INFINITY) {
            m = wave_max_f(tmax);
        } else if (__any(tmax > m + kRescale)) {
            const float mn = wave_max_f(tmax);
            const float alpha = exp2f(m - mn);
#pragma unroll
            for (int j = 0; j < 32; ++j) acc[j] *= alpha;
            zacc *= alpha;
            lsum *= alpha;
            m = mn;
        }
        const float m24 = m - 24.0f;
#pragma unroll
        for (int s = 0; s < UPR; ++s) {
            if (valid[s]) {
                const float p = exp2_for_asm(sc[s] - m24);  // read by the mix asm below
                lsum += p;
                zacc = mix_hi(vmw[s], p, zacc);
                ValueAxpy f{mix_lo(vmw[s], p, 0.f), acc};
                Unit<BV>::visit(vw[s], f);
            }
        }
    };

    // Key scores of one super-tile; `full` means every token is a quantized key.
    auto key_scores = [&](int st, const St& r, bool full, float (&sc)[UPR], bool (&valid)[UPR]) {
        const int b0 = st >> lgk;
#pragma unroll
        for (int bl = 0; bl < 2; ++bl) {
            if (bl == 0 || (two_blocks && ((b0 + 1) << lgk) < qend)) {
                float qsv[KPL];
                float pz = 0.f;
#pragma unroll
                for (int k = 0; k < KPL; ++k) {
                    qsv[k] = mix_lo(r.kmw[bl][k], qks[k], 0.f);
                    pz = mix_hi(r.kmw[bl][k], qk[k], pz);
                }
                store_lds_n<KPL>(&qs_lds[wave][bl][((KPL * lane) >> 5) * QSP + ((KPL * lane) & 31)], qsv);
                pz = unit_sum<32 / KPL>(pz);
                if ((lane & (32 / KPL - 1)) == 0) bz_lds[wave][bl][(KPL * lane) >> 5] = pz;
            }
        }
        wave_sync_lds();
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int bl = two_blocks ? h : 0;
            float qv[32];
            const float4* src = (const float4*)&qs_lds[wave][bl][cg * QSP];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const float4 v = src[k];
                qv[4 * k] = v.x;
                qv[4 * k + 1] = v.y;
                qv[4 * k + 2] = v.z;
                qv[4 * k + 3] = v.w;
            }
            const float bzv = bz_lds[wave][bl][cg];
            if (HALF % 2 == 0 && full) {
#pragma unroll
                for (int s = h * HALF; s + 1 < (h + 1) * HALF; s += 2) {
                    KeyDot2 f{qv, bzv, 0.f, bzv, 0.f};
                    Unit<BK>::visit2(r.kw[s], r.kw[s + 1], f);
                    sc[s] = group_sum<UPR>(f.a0 + f.a1);
                    sc[s + 1] = group_sum<UPR>(f.b0 + f.b1);
                    valid[s] = valid[s + 1] = true;
                }
            } else {
#pragma unroll
                for (int s = h * HALF; s < (h + 1) * HALF; ++s) {
                    valid[s] = st + s * TPW + ts < qend;
                    float part = 0.f;
                    if (valid[s]) {
                        KeyDot f{qv, bzv, 0.f};
                        Unit<BK>::visit(r.kw[s], f);
                        part = f.a0 + f.a1;
                    }
                    part = group_sum<UPR>(part);
                    sc[s] = valid[s] ? part : -INFINITY;
                }
            }
        }
        wave_sync_lds();  // qs_lds is rewritten by the next super-tile
    };

    // Rotary keys: per 32-token half h, the weights of the lane's prologue
    // pairs from the query rotated to the half's first position st + 32h (the
    // second half's angle is the first's plus the table's row 32).
    auto key_scores_rope = [&](int st, const St& r, float (&sc)[UPR], bool (&valid)[UPR]) {
        float ca[KPP], sa[KPP];
#pragma unroll
        for (int k = 0; k < KPP; ++k) rope_cs(st, th[k], ca[k], sa[k]);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int bl = two_blocks ? h : 0;
#pragma unroll
            for (int k = 0; k < KPP; ++k) {
                const int pp = lane + 64 * k;
                if (h == 1) {
                    const float2 r32 = *(const float2*)&rt_lds[rope_lds_off(min(pp, D / 2 - 1), 32)];
                    const float c1 = fmaf(ca[k], r32.x, -(sa[k] * r32.y));
                    sa[k] = fmaf(sa[k], r32.x, ca[k] * r32.y);
                    ca[k] = c1;
                }
                if (pp < D / 2) {
                    const float qa = q_lds[pp], qb = q_lds[pp + D / 2];
                    const float Qa = fmaf(ca[k], qa, sa[k] * qb), Qb = fmaf(ca[k], qb, -(sa[k] * qa));
                    const uint32_t ma = r.kmw[bl][2 * k], mb = r.kmw[bl][2 * k + 1];
                    const float f = (float)(1 << (24 - code_shift<BK>(pp & 15)));
                    const float s_a = f16_to_f32(ma & 0xffffu) * f, z_a = f16_to_f32(ma >> 16);
                    const float s_b = f16_to_f32(mb & 0xffffu) * f, z_b = f16_to_f32(mb >> 16);
                    const int slot = pp + (pp >> 4);
                    pw4_lds[wave][h][slot] = make_float4(Qa * s_a, Qb * s_b, fmaf(Qa, z_a, Qb * z_b), Qb * s_a);
                    pw2_lds[wave][h][slot] = make_float2(-(Qa * s_b), fmaf(Qb, z_a, -(Qa * z_b)));
                }
            }
        }
        wave_sync_lds();
#pragma unroll
        for (int s = 0; s < UPR; ++s) valid[s] = st + s * TPW + ts < qend;
        if constexpr (HALF >= 2) {  // the two tokens s, s + 1 of a half share the pair weights
#pragma unroll
            for (int s = 0; s < UPR; s += 2) {
                const int h = s / HALF, u = (s - h * HALF) * TPW + ts;
                RopeDot2 f{&pw4_lds[wave][h][17 * cg], &pw2_lds[wave][h][17 * cg],
                           &rt_lds[rope_lds_off(16 * cg, u)], &rt_lds[rope_lds_off(16 * cg, u + TPW)],
                           0.f, 0.f, 0.f, 0.f};
                visit_runs2<BK>(r.kw[s], r.kw[s + 1], (16 * BK * cg) & 31, f);
                const float p0 = group_sum<UPR>(f.a0 + f.a1), p1 = group_sum<UPR>(f.b0 + f.b1);
                sc[s] = valid[s] ? p0 : -INFINITY;
                sc[s + 1] = valid[s + 1] ? p1 : -INFINITY;
                __builtin_amdgcn_sched_barrier(0);  // one token pair's weights live at a time
            }
        } else {
#pragma unroll
            for (int s = 0; s < UPR; ++s) {
                const int h = s / HALF, u = (s - h * HALF) * TPW + ts;
                RopeDot f{&pw4_lds[wave][h][17 * cg], &pw2_lds[wave][h][17 * cg],
                          &rt_lds[rope_lds_off(16 * cg, u)], 0.f, 0.f};
                visit_runs<BK>(r.kw[s], (16 * BK * cg) & 31, f);
                const float part = group_sum<UPR>(f.a0 + f.a1);
                sc[s] = valid[s] ? part : -INFINITY;
                __builtin_amdgcn_sched_barrier(0);  // one token's weights live at a time
            }
        }
        wave_sync_lds();  // the weights are rewritten by the next super-tile
    };

    // Rotary full-precision rows: per half h, the query pairs rotated to the
    // anchors t0 + 32h (x, y) and t0 + off + 32h (z, w).
    auto rope_queries = [&](int t0, int off) {
#pragma unroll
        for (int k = 0; k < KPP; ++k) {
            const int pp = lane + 64 * k;
            float c0, s0, c1, s1;
            rope_cs(t0, th[k], c0, s0);
            rope_cs(t0 + off, th[k], c1, s1);
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                if (h == 1) {
                    const float2 r32 = *(const float2*)&rt_lds[rope_lds_off(min(pp, D / 2 - 1), 32)];
                    float t = fmaf(c0, r32.x, -(s0 * r32.y));
                    s0 = fmaf(s0, r32.x, c0 * r32.y);
                    c0 = t;
                    t = fmaf(c1, r32.x, -(s1 * r32.y));
                    s1 = fmaf(s1, r32.x, c1 * r32.y);
                    c1 = t;
                }
                if (pp < D / 2) {
                    const float qa = q_lds[pp], qb = q_lds[pp + D / 2];
                    pw4_lds[wave][h][pp + (pp >> 4)] = make_float4(fmaf(c0, qa, s0 * qb), fmaf(c0, qb, -(s0 * qa)),
                                                                   fmaf(c1, qa, s1 * qb), fmaf(c1, qb, -(s1 * qa)));
                }
            }
        }
        wave_sync_lds();
    };

    auto compute_stage = [&](int st, const St& r) {
        float sc[UPR];
        bool valid[UPR];
        if constexpr (ROPE) {
            key_scores_rope(st, r, sc, valid);
        } else if (st + 64 <= qend) {
            key_scores(st, r, true, sc, valid);
        } else {
            key_scores(st, r, false, sc, valid);
        }
        softmax_and_values(sc, r.vw, r.vmw, valid);
    };

    // ---- quantized keys: super-tiles of 64 tokens interleaved across waves,
    // a ring of NS register stages keeps NS-1 super-tiles in flight
    if (st0 < qend) {
        St rg[NS];
        int st = st0;
#pragma unroll
        for (int i = 0; i < NS - 1; ++i) load_stage(st + i * STEP, rg[i]);
        bool more = true;
        while (more) {
#pragma unroll
            for (int i = 0; i < NS; ++i) {
                if (more) {
                    load_stage(st + (NS - 1) * STEP, rg[(i + NS - 1) % NS]);
                    compute_stage(st, rg[i]);
                    st += STEP;
                    more = st < qend;
                }
            }
        }
    }

    // ---- residual keys (input dtype), fewer than G tokens, one wave
    if (appended) __syncthreads();  // the step's new rows are in place (residual and window rows)
    if (wave == 0) {
        for (int st = max(wa, nqk); st < wb; st += 64) {
            uint32_t vw[UPR][BV], vmw[UPR];
            float sc[UPR];
            bool valid[UPR];
            if constexpr (ROPE) rope_queries(st, 0);
            // loads are unconditional, from the clamped token (a load under a
            // branch waits on its own), so they can be issued ahead of the sums
#pragma unroll
            for (int s = 0; s < UPR; ++s) {
                const int t = st + s * TPW + ts;
                valid[s] = t < wb;
                const int tc = valid[s] ? t : wb - 1;
                const PageRow pr = page_row(a.pages, e, tc);
                load_words<BV>((const uint32_t*)(vc + pr.base + (size_t)pr.row * (D * BV / 8)) + cg * BV, vw[s]);
                vmw[s] = ((const uint32_t*)(vm + pr.base))[(size_t)pr.row * vgpr + vg];
                float part = 0.f;
                if constexpr (ROPE) {
                    const size_t base = (size_t)(tc & ((1 << lgk) - 1)) * D + 16 * cg;
                    float xa[16], xb[16];
                    load16_rt(kr, base, a.in_dtype, xa);
                    load16_rt(kr, base + D / 2, a.in_dtype, xb);
                    const int h = s / HALF, u = (s - h * HALF) * TPW + ts;
                    part = rope_row_score(&pw4_lds[wave][h][17 * cg], false, &rt_lds[rope_lds_off(16 * cg, u)],
                                          xa, xb);
                } else {
                    const size_t base = (size_t)(tc & ((1 << lgk) - 1)) * D + 32 * cg;
                    float x[32];
                    if (a.in_dtype == 0) load32<0>(kr, base, x);
                    else if (a.in_dtype == 1) load32<1>(kr, base, x);
                    else load32<2>(kr, base, x);
#pragma unroll
                    for (int j = 0; j < 32; ++j) part = fmaf(q_lds[32 * cg + j], x[j], part);
                }
                part = group_sum<UPR>(part);
                sc[s] = valid[s] ? part : -INFINITY;
            }
            softmax_and_values(sc, vw, vmw, valid);
            if constexpr (ROPE) wave_sync_lds();  // the next tile rewrites the rotated queries
        }
    }

    // ---- full-precision window and sinks (last split): keys and values in the
    // input dtype from the window area, 64-token super-tiles across the waves.
    // A value row enters acc[j] as p * v_j * 2^(code_shift(j) - 24), which the
    // code-shift undo below turns into p * v_j.
    if (a.win_mode && split == nsplit - 1) {
        const int nfp = fp_count(a, len, te);
        const uint8_t* kwn = a.resid + e.resid[0] + (size_t)kvh * e.resid_hs[0] + a.win_off[0];
        const uint8_t* vwn = a.resid + e.resid[1] + (size_t)kvh * e.resid_hs[1] + a.win_off[1];
        auto row32 = [&](const uint8_t* base, size_t off, float (&x)[32]) {
            if (a.in_dtype == 0) load32<0>(base, off, x);
            else if (a.in_dtype == 1) load32<1>(base, off, x);
            else load32<2>(base, off, x);
        };
        // rotary positions: i for the sinks (i < ns), i + rs - ns after them
        const int ns = min(len, a.sinks), rs = max(te, ns);
        for (int st = 64 * wave; st < nfp; st += 64 * NW) {
            float sc[UPR];
            bool valid[UPR];
            int rows[UPR];
            if constexpr (ROPE) rope_queries(st, rs - ns);
#pragma unroll
            for (int s = 0; s < UPR; ++s) {
                const int i = st + s * TPW + ts;
                valid[s] = i < nfp;
                rows[s] = valid[s] ? window_row(fp_token(a, len, te, i), a.sinks, a.win_rows, e.ring) : 0;
                float part = 0.f;
                if constexpr (ROPE) {
                    float xa[16], xb[16];
                    load16_rt(kwn, (size_t)rows[s] * D + 16 * cg, a.in_dtype, xa);
                    load16_rt(kwn, (size_t)rows[s] * D + D / 2 + 16 * cg, a.in_dtype, xb);
                    const int h = s / HALF, u = (s - h * HALF) * TPW + ts;
                    part = rope_row_score(&pw4_lds[wave][h][17 * cg], i >= ns, &rt_lds[rope_lds_off(16 * cg, u)],
                                          xa, xb);
                } else {
                    float x[32];
                    row32(kwn, (size_t)rows[s] * D + 32 * cg, x);
#pragma unroll
                    for (int j = 0; j < 32; ++j) part = fmaf(q_lds[32 * cg + j], x[j], part);
                }
                part = group_sum<UPR>(part);
                sc[s] = valid[s] ? part : -INFINITY;
            }
            float tmax = sc[0];
#pragma unroll
            for (int s = 1; s < UPR; ++s) tmax = fmaxf(tmax, sc[s]);
            const float mn = wave_max_f(tmax);
            if (mn > m) {  // exact maximum here: this loop runs once per split
                const float alpha = m == -INFINITY ? 0.f : exp2f(m - mn);
#pragma unroll
                for (int j = 0; j < 32; ++j) acc[j] *= alpha;
                zacc *= alpha;
                lsum *= alpha;
                m = mn;
            }
            const float m24 = m - 24.0f;
#pragma unroll
            for (int s = 0; s < UPR; ++s) {
                float v[32];
                row32(vwn, (size_t)rows[s] * D + 32 * cg, v);  // unconditional: invalid rows are not used
                if (valid[s]) {
                    const float p = __builtin_amdgcn_exp2f(sc[s] - m24);
                    lsum += p;
#pragma unroll
                    for (int j = 0; j < 32; ++j)
                        acc[j] = fmaf(p * ((float)(1 << code_shift<BV>(j)) * (1.0f / 16777216.0f)), v[j], acc[j]);
                }
            }
            if constexpr (ROPE) wave_sync_lds();  // the next tile rewrites the rotated queries
        }
    }

    // ---- wave result: undo the code shifts, add the zero-point sums, reduce over tokens
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = acc[j] * (float)(1 << (24 - code_shift<BV>(j))) + zacc;
#pragma unroll
    for (int off = UPR; off < 64; off <<= 1) {
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[j] += __shfl_xor(acc[j], off);
        lsum += __shfl_xor(lsum, off);
    }
    if (ts == 0) {
#pragma unroll
        for (int j = 0; j < 32; ++j) mrg_o[wave][32 * cg + j] = acc[j];
    }
    if (lane == 0) {
        mrg_ml[wave][0] = m;
        mrg_ml[wave][1] = lsum;
    }
    __syncthreads();

    // ---- merge the NW waves; several splits are merged by merge_kernel
    float M = -INFINITY;
#pragma unroll
    for (int w = 0; w < NW; ++w) M = fmaxf(M, mrg_ml[w][0]);
    float L = 0.f, wgt[NW];
#pragma unroll
    for (int w = 0; w < NW; ++w) {
        wgt[w] = mrg_ml[w][0] == -INFINITY ? 0.f : exp2f(mrg_ml[w][0] - M);
        L = fmaf(mrg_ml[w][1], wgt[w], L);
    }
    const size_t slot = ((size_t)seq * a.q_heads + kvh) * a.max_chunks + split;
    const float inv = 1.0f / L;
    for (int c = tid; c < D; c += NT) {
        float o = 0.f;
#pragma unroll
        for (int w = 0; w < NW; ++w) o = fmaf(mrg_o[w][c], wgt[w], o);
        if (nsplit == 1) out[c] = o * inv;
        else a.ws_o[slot * D + c] = o;
    }
    if (nsplit > 1 && tid == 0) {
        a.ws_ml[slot * 2 + 0] = M;
        a.ws_ml[slot * 2 + 1] = L;
    }
}

// 4 waves per workgroup with a 3-stage register ring measured fastest on the
// Llama-2-7B-shaped step (6 waves with 2 stages was ~20% slower); the rotary
// instantiations keep 2 stages (3 measured slower and spill at 8 bits).
#if KVQ_MHA_ROPE
constexpr bool kRope = true;
constexpr int kStages = 2;
#else
constexpr bool kRope = false;
constexpr int kStages = 3;
#endif

// Whether the fused instantiation (a few more registers) keeps the plain
// one's resident workgroups per compute unit; asked once per bit pair.
template <int D, int BK, int BV>
bool fused_keeps_occupancy() {
    static int cached = -1;  // racing first calls compute the same value
    if (cached < 0) {
        int plain = 0, fused = 0;
        const bool ok = hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &plain, (const void*)decode_mha_kernel<D, BK, BV, 4, kStages, false, kRope>, 4 * 64, 0) ==
                            hipSuccess &&
                        hipOccupancyMaxActiveBlocksPerMultiprocessor(
                            &fused, (const void*)decode_mha_kernel<D, BK, BV, 4, kStages, true, kRope>, 4 * 64, 0) ==
                            hipSuccess;
        cached = ok && fused >= plain ? 1 : 0;
    }
    return cached == 1;
}

template <int D, int BK>
bool fused_ok_bv(int bv) {
    switch (bv) {
        case 2: return fused_keeps_occupancy<D, BK, 2>();
        case 3: return fused_keeps_occupancy<D, BK, 3>();
        case 4: return fused_keeps_occupancy<D, BK, 4>();
        case 6: return fused_keeps_occupancy<D, BK, 6>();
        default: return fused_keeps_occupancy<D, BK, 8>();
    }
}

template <int D, int BK, int BV>
hipError_t launch_nw(const DecodeArgs& a, dim3 grid, hipStream_t s) {
    if (a.append_fused)
        hipLaunchKernelGGL((decode_mha_kernel<D, BK, BV, 4, kStages, true, kRope>), grid, dim3(4 * 64), 0, s, a);
    else hipLaunchKernelGGL((decode_mha_kernel<D, BK, BV, 4, kStages, false, kRope>), grid, dim3(4 * 64), 0, s, a);
    return hipGetLastError();
}

template <int D, int BK>
hipError_t launch_bv(const DecodeArgs& a, int bv, dim3 grid, hipStream_t s) {
    switch (bv) {
        case 2: return launch_nw<D, BK, 2>(a, grid, s);
        case 3: return launch_nw<D, BK, 3>(a, grid, s);
        case 4: return launch_nw<D, BK, 4>(a, grid, s);
        case 6: return launch_nw<D, BK, 6>(a, grid, s);
        default: return launch_nw<D, BK, 8>(a, grid, s);
    }
}

template <int D>
hipError_t launch_bk(const DecodeArgs& a, int bk, int bv, dim3 grid, hipStream_t s) {
    switch (bk) {
        case 2: return launch_bv<D, 2>(a, bv, grid, s);
        case 3: return launch_bv<D, 3>(a, bv, grid, s);
        case 4: return launch_bv<D, 4>(a, bv, grid, s);
        case 6: return launch_bv<D, 6>(a, bv, grid, s);
        default: return launch_bv<D, 8>(a, bv, grid, s);
    }
}

}  // namespace

// This file is compiled once per head_dim (KVQ_MHA_HEAD_DIM = 64, 128, 256),
// plain and with KVQ_MHA_ROPE = 1 (the rotary instantiations).
#define KVQ_CAT2(a, b) a##b
#define KVQ_CAT(a, b) KVQ_CAT2(a, b)
#if !KVQ_MHA_ROPE
#define KVQ_MHA_FUSED_OK KVQ_CAT(mha_fused_ok_d, KVQ_MHA_HEAD_DIM)
#define KVQ_MHA_LAUNCH KVQ_CAT(launch_decode_mha_d, KVQ_MHA_HEAD_DIM)
#else
#define KVQ_MHA_FUSED_OK KVQ_CAT(mha_rope_fused_ok_d, KVQ_MHA_HEAD_DIM)
#define KVQ_MHA_LAUNCH KVQ_CAT(launch_decode_mha_rope_d, KVQ_MHA_HEAD_DIM)
#endif
bool KVQ_MHA_FUSED_OK(int bits_k, int bits_v) {
    constexpr int D = KVQ_MHA_HEAD_DIM;
    switch (bits_k) {
        case 2: return fused_ok_bv<D, 2>(bits_v);
        case 3: return fused_ok_bv<D, 3>(bits_v);
        case 4: return fused_ok_bv<D, 4>(bits_v);
        case 6: return fused_ok_bv<D, 6>(bits_v);
        default: return fused_ok_bv<D, 8>(bits_v);
    }
}

hipError_t KVQ_MHA_LAUNCH(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s) {
    // x: the quantized splits only (the workspace's full-precision slots have no
    // workgroups here: empty ones would leave the busy ones on a few XCDs)
    dim3 grid(a.max_chunks - a.win_splits, a.kv_heads, nseqs * a.n_layers);
    return launch_bk<KVQ_MHA_HEAD_DIM>(a, bits_k, bits_v, grid, s);
}

}  // namespace kvq
