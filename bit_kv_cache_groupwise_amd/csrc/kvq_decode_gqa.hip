// Decode attention for query groups (q_heads / kv_heads = R >= 2): the R
// queries that share a kv head turn the decode step into a small dense
// contraction, so both products run on MFMA (v_mfma_f32_16x16x32_f16) with
// the packed codes as exact fp16 operands. Keys on the channel axis, values on
// the token axis.
//
// Sources, by page title and section:
//   [N] nalar.dev, "Kuantisasi KV cache untuk mengurangi memory inferensi
//       long-context", "Kuantisasi dapat memindahkan pekerjaan ke decode path"
//       (unpack and apply the scales inside the attention kernel)
//   [N] same page, "Ukuran cache bertambah mengikuti token, layer, dan KV head"
//       (grouped-query attention shares kv heads among query heads)
//   [U] unite.ai (pt), "Por Que o Cache KV E Onde Isso Morde" (decode reads the
//       whole cache once per generated token)
//
// Work decomposition: workgroup = (split of the token axis, (kv head, group of
// up to 16 of its query heads), seq), 4 waves. The waves take interleaved
// 32-token tiles and never exchange data inside the loop: each keeps its own
// running maximum, denominator and output rows for the 16 query rows (zero
// padded), and the four are merged once at the end, in LDS, in a fixed order.
//
// Per tile and wave (lane l: n = l % 16, g = l / 16):
//   scores^T[t][r] = 2^16 sum_c A[t][c] B[c][r] + bias[r]
//     A = key codes of token t as fp16 values (code << sh) 2^-24, unpacked from
//         the lane's own row words (exact); lane group g holds a quarter of
//         the channels, of token rows t0 + 8(m >> 2) + 4h + (m & 3) (h = 0, 1);
//     B = q'_rc s_c in fp16 hi + lo parts (two MFMAs), q' = q * softmax scale *
//         log2(e) * 2^(8 - sh), built per tile from q' in LDS and the block's
//         steps staged in LDS; bias[r] = sum_c q'_rc z_c on the VALU;
//   the score layout (lane: query n, 8 consecutive tokens 8g..8g+7) is the
//   A-operand layout of the value product, so softmax weights stay in place;
//   O[r][c] += 2^(24-kb-vsh) sum_t (2^kb p_rt s_t,g(c))[hi + lo] V[t][c],
//     V = value codes of the tile staged in LDS as one byte per code
//         [token][channel]; ds_read_b64_tr_b8 hands lane n the tokens
//         8g..8g+7 of one channel (the B-operand layout), and v_perm turns two
//         bytes into two fp16 (code << vsh) 2^-24;
//   Z[r][k] += 2^-KZ sum_t (2^KZ p_rt)[hi + lo] (z_t,k | 1): zero-point sums per
//     value group and, in the column after the last group, the denominator.
//
// Softmax: online in the log2 domain with the exact running maximum, so weights
// are <= 1. They enter the fp16 operands pre-scaled by powers of two: 2^kb for
// p * s (kb per query row, from BV + 2: lowered per tile when large value
// steps would push 2^kb p s past 2^15, and set from the row's largest p s over
// the tile, up to 15, when a small step would take its products below fp16's
// normal range; the row's accumulators are rescaled exactly), 2^KZ for the
// zero points. q' is kept below 2^14 by a power of two per workgroup, and the key
// weights q' s of a block whose steps would push them past 2^15 are scaled by
// 2^-f. Splits are merged by merge_kernel.
//
// Keys cached before the rotary embedding ([U] "Embebedos Rotatorios
// Complicam as Chaves": rotate after dequantization; objects built with
// KVQ_GQA_ROPE): lane group g holds D/8 whole channel pairs (i, i + D/2), a
// run of codes and its partner run. Per tile and pair the lane reconstructs
// its token's two key values (one v_fma_mix each from the code halves), rotates
// them by the token's offset u in the tile ((cos, sin)(u theta_i) held in
// registers: the lane's offsets never change), and splits them into fp16
// hi + lo parts: A. B is q' rotated back to the tile's first position, also
// hi + lo, so the score takes three MFMAs per chunk (hi hi, hi lo, lo hi).
// The zero points are inside the reconstructed keys (no bias term).
//
// Pipeline: one tile of codes and metadata in registers per wave: the value and
// metadata words of tile i + 4 are requested as soon as tile i's are staged in
// LDS, its key words as soon as tile i's key products are issued.
#include <utility>

#include "kvq_device.h"
#include "kvq_internal.h"

#ifndef KVQ_GQA_ROPE
#define KVQ_GQA_ROPE 0
#endif

namespace kvq {
namespace {

using namespace dev;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef int i32x2_t __attribute__((ext_vector_type(2)));

union Frag {
    half8_t h;
    uint32_t u[4];
};

__device__ __forceinline__ f32x4 mfma(const Frag& a, const Frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.h, b.h, c, 0, 0, 0);
}

// v_fma_mix_f32 with the first operand an fp16 half of a word: exact product
// of an fp16 and an fp32 value, one rounding.
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
// x - half(h): exact when half(h) is x truncated to fp16 (Sterbenz).
__device__ __forceinline__ float rem_lo(uint32_t h, float x) {
    float d;
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(x));
    return d;
}
__device__ __forceinline__ float rem_hi(uint32_t h, float x) {
    float d;
    asm("v_fma_mix_f32 %0, %1, -1.0, %2 op_sel:[1,0,0] op_sel_hi:[1,0,0]" : "=v"(d) : "v"(h), "v"(x));
    return d;
}
__device__ __forceinline__ uint32_t pk_rtz(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_pkrtz(a, b));
}
// a * half_S(b) - half_S(c), one rounding (S selects the low or high halves).
__device__ __forceinline__ float mix3_lo(float a, uint32_t b, uint32_t c) {
    float d;
    asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,0,0] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}
__device__ __forceinline__ float mix3_hi(float a, uint32_t b, uint32_t c) {
    float d;
    asm("v_fma_mix_f32 %0, %1, %2, -%3 op_sel:[0,1,1] op_sel_hi:[0,1,1]" : "=v"(d) : "v"(a), "v"(b), "v"(c));
    return d;
}
typedef _Float16 half2_t __attribute__((ext_vector_type(2)));
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pk_mul(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_bit_cast(half2_t, a) * __builtin_bit_cast(half2_t, b));
}
// (a0, a1) * (s0, s1) as hi + lo fp16 pairs: hi = fp16 product of the fp16
// pair ah ~= (a0, a1) and s; lo = fp16 of the exact rest a * s - hi.
__device__ __forceinline__ void mul_split(uint32_t ah, float a0, float a1, uint32_t sp, uint32_t& hi, uint32_t& lo) {
    hi = pk_mul(ah, sp);
    lo = pk_rtz(mix3_lo(a0, sp, hi), mix3_hi(a1, sp, hi));
}
// (x0, x1) ~= hi + lo with hi = fp16 truncation and lo = fp16 of the exact rest.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    hi = pk_rtz(x0, x1);
    lo = pk_rtz(rem_lo(hi, x0), rem_hi(hi, x1));
}

// Integer codes enter the MFMAs as fp16 values (code << sh) 2^-24: subnormals,
// or normals of exponent 1, where the value is still linear in the bit pattern
// (below 2048). The MFMA's sum of products loses low bits of products whose
// subnormal operand uses only the bottom of the mantissa, so every code is
// shifted until its top bit reaches mantissa bit 9 or 10.
__host__ __device__ constexpr int key_shift(int B) { return B == 2 ? 9 : B == 3 ? 8 : B == 4 ? 7 : B == 6 ? 5 : 3; }
// Value codes come out of LDS one byte each; 2- and 3-bit codes go to the high
// byte of a half (one v_perm per pair, no shift).
__host__ __device__ constexpr int val_shift(int B) { return B <= 3 ? 8 : B == 4 ? 7 : B == 6 ? 5 : 3; }

// Key-code fragments: 8-code chunk K of a lane's code range as 8 fp16 halves.
// Half j of the fragment holds code 8K + PERM[j] of the range as code << key_shift(B).
template <int B>
struct KeyFrag;

template <>
struct KeyFrag<2> {
    static constexpr int PERM[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    template <int K>
    static __device__ __forceinline__ void get(const uint32_t* w, Frag& f) {
        // the chunk's two bytes (4 codes each) to the low byte of each half
        const uint32_t x = w[K / 2];
        const uint32_t y = (K & 1) ? __builtin_amdgcn_perm(x, x, 0x0c030c02u) : __builtin_amdgcn_perm(x, x, 0x0c010c00u);
        f.u[0] = (y << 9) & 0x06000600u;
        f.u[1] = (y << 7) & 0x06000600u;
        f.u[2] = (y << 5) & 0x06000600u;
        f.u[3] = (y << 3) & 0x06000600u;
    }
};

template <>
struct KeyFrag<4> {
    static constexpr int PERM[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    template <int K>
    static __device__ __forceinline__ void get(const uint32_t* w, Frag& f) {
        const uint32_t x = w[K];  // nibble i of each half to bits 7..10
        f.u[0] = (x << 7) & 0x07800780u;
        f.u[1] = (x << 3) & 0x07800780u;
        f.u[2] = (x >> 1) & 0x07800780u;
        f.u[3] = (x >> 5) & 0x07800780u;
    }
};

template <>
struct KeyFrag<8> {
    static constexpr int PERM[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    template <int K>
    static __device__ __forceinline__ void get(const uint32_t* w, Frag& f) {
        const uint32_t x0 = w[2 * K], x1 = w[2 * K + 1];  // bytes to bits 3..10 of the halves
        f.u[0] = (x0 << 3) & 0x07f807f8u;
        f.u[1] = (x0 >> 5) & 0x07f807f8u;
        f.u[2] = (x1 << 3) & 0x07f807f8u;
        f.u[3] = (x1 >> 5) & 0x07f807f8u;
    }
};

// Rotary layout: the words of a run of N codes (N = D/8 = 16 or 32); a run of
// 16 3-bit codes starts on a half word when g is odd (two words, aligned at use).
template <int B, int N>
__host__ __device__ constexpr int rope_run_words() { return N == 32 ? B : (B == 3 ? 2 : B / 2); }
// Bit at which pair jj (0..3) of a chunk sits in its fp16 half after extraction.
template <int B>
__host__ __device__ constexpr int rope_code_shift(int jj) { return B == 2 ? 2 * jj : B == 4 ? 4 * (jj & 1) : 0; }

// Code j (0..31) of one packed 32-channel unit (little-endian bitstream).
template <int B, int J>
__device__ __forceinline__ uint32_t unit_code(const uint32_t* w) {
    constexpr int pos = J * B, wi = pos >> 5, sh = pos & 31;
    if constexpr (sh + B <= 32) return (w[wi] >> sh) & ((1u << B) - 1u);
    else return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << B) - 1u);
}

// Codes 4C + jj (jj = 0..3) of run A (wa) and run B (wb) as the words
// (a | b << 16) << rope_code_shift(jj): fp16 halves (code << sh) 2^-24.
template <int B, int C>
__device__ __forceinline__ void rope_chunk_codes(const uint32_t* wa, const uint32_t* wb, uint32_t (&ab)[4]) {
    // v_perm selector: byte k of run A to byte 0, byte k of run B to byte 2
    auto sel = [](uint32_t k) { return k | 0x0c00u | ((4u + k) << 16) | 0x0c000000u; };
    if constexpr (B == 8) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) ab[jj] = __builtin_amdgcn_perm(wb[C], wa[C], sel(jj));
    } else if constexpr (B == 4) {
        constexpr uint32_t b0 = 2 * (C % 2);  // the byte of codes 4C, 4C + 1
        const uint32_t lo = __builtin_amdgcn_perm(wb[C / 2], wa[C / 2], sel(b0));
        const uint32_t hi = __builtin_amdgcn_perm(wb[C / 2], wa[C / 2], sel(b0 + 1));
        ab[0] = lo & 0x000f000fu;
        ab[1] = lo & 0x00f000f0u;
        ab[2] = hi & 0x000f000fu;
        ab[3] = hi & 0x00f000f0u;
    } else if constexpr (B == 2) {
        const uint32_t v = __builtin_amdgcn_perm(wb[C / 4], wa[C / 4], sel(C % 4));
        ab[0] = v & 0x00030003u;
        ab[1] = v & 0x000c000cu;
        ab[2] = v & 0x00300030u;
        ab[3] = v & 0x00c000c0u;
    } else {  // 3 and 6 bits: one extract per code
        static_for<4>([&](auto JJ) {
            constexpr int j = 4 * C + JJ;
            ab[JJ] = unit_code<B, j>(wa) | (unit_code<B, j>(wb) << 16);
        });
    }
}

// 3- and 6-bit codes straddle words: one bit-field extract per code.
template <int B>
struct KeyFragStraddle {
    static constexpr int PERM[8] = {0, 1, 2, 3, 4, 5, 6, 7};
    static constexpr int SH = key_shift(B);
    template <int K>
    static __device__ __forceinline__ void get(const uint32_t* w, Frag& f) {
        // chunk K covers codes 8K..8K+7 of the lane's range; a 32-code unit is B words
        const uint32_t* u = w + (K / 4) * B;
        constexpr int j0 = 8 * (K % 4);
        f.u[0] = (unit_code<B, j0 + 0>(u) << SH) | (unit_code<B, j0 + 1>(u) << (16 + SH));
        f.u[1] = (unit_code<B, j0 + 2>(u) << SH) | (unit_code<B, j0 + 3>(u) << (16 + SH));
        f.u[2] = (unit_code<B, j0 + 4>(u) << SH) | (unit_code<B, j0 + 5>(u) << (16 + SH));
        f.u[3] = (unit_code<B, j0 + 6>(u) << SH) | (unit_code<B, j0 + 7>(u) << (16 + SH));
    }
};
template <>
struct KeyFrag<3> : KeyFragStraddle<3> {};
template <>
struct KeyFrag<6> : KeyFragStraddle<6> {};

// One 32-channel value unit as 32 bytes (8 words), one code per byte. Byte
// position p of the unit holds channel val_chan<B>(p).
template <int B>
__device__ __forceinline__ void unit_to_bytes(const uint32_t* w, uint32_t* out) {
    if constexpr (B == 8) {
#pragma unroll
        for (int k = 0; k < 8; ++k) out[k] = w[k];
    } else if constexpr (B == 4) {
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            out[2 * k] = w[k] & 0x0f0f0f0fu;
            out[2 * k + 1] = (w[k] >> 4) & 0x0f0f0f0fu;
        }
    } else if constexpr (B == 2) {
#pragma unroll
        for (int k = 0; k < 2; ++k) {
            out[4 * k + 0] = w[k] & 0x03030303u;
            out[4 * k + 1] = (w[k] >> 2) & 0x03030303u;
            out[4 * k + 2] = (w[k] >> 4) & 0x03030303u;
            out[4 * k + 3] = (w[k] >> 6) & 0x03030303u;
        }
    } else {
        static_for<8>([&](auto K) {
            constexpr int k = K;
            out[k] = unit_code<B, 4 * k>(w) | (unit_code<B, 4 * k + 1>(w) << 8) | (unit_code<B, 4 * k + 2>(w) << 16) |
                     (unit_code<B, 4 * k + 3>(w) << 24);
        });
    }
}
template <int B>
__device__ __forceinline__ int val_chan(int p) {
    if constexpr (B == 4) return (p & ~7) + 2 * (p & 3) + ((p >> 2) & 1);
    else if constexpr (B == 2) return (p & ~15) + 4 * (p & 3) + ((p >> 2) & 3);
    else return p;
}

// N consecutive words from p, whose byte address is a multiple of ALIGN.
template <int N, int ALIGN>
__device__ __forceinline__ void load_n(const uint32_t* p, uint32_t* w) {
    if constexpr (ALIGN >= 16 && N % 4 == 0) {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) {
            const uint4 v = ((const uint4*)p)[k];
            w[4 * k] = v.x, w[4 * k + 1] = v.y, w[4 * k + 2] = v.z, w[4 * k + 3] = v.w;
        }
    } else if constexpr (ALIGN >= 8 && N % 2 == 0) {
#pragma unroll
        for (int k = 0; k < N / 2; ++k) {
            const uint2 v = ((const uint2*)p)[k];
            w[2 * k] = v.x, w[2 * k + 1] = v.y;
        }
    } else {
#pragma unroll
        for (int k = 0; k < N; ++k) w[k] = p[k];
    }
}

constexpr int pow2_align(int bytes) { return (bytes & 15) == 0 ? 16 : (bytes & 7) == 0 ? 8 : (bytes & 3) == 0 ? 4 : 1; }
constexpr int min_align(int a, int b) { return a < b ? a : b; }

// Sums and maxima over the 4 lanes that share l % 16 (lanes l, l^16, l^32, l^48),
// with the row-swap permutes.
__device__ __forceinline__ float col4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}
__device__ __forceinline__ float col4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}

// LDS writes of this wave visible to this wave (each wave owns its tile areas).
__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}
__device__ __forceinline__ void wg_lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Largest value over the wave of a BITS-bit unsigned field (scalar result:
// binary search over ballots).
template <int BITS>
__device__ __forceinline__ int wave_max_field(int e) {
    int emax = 0;
#pragma unroll
    for (int b = 1 << (BITS - 1); b; b >>= 1)
        if (__builtin_amdgcn_ballot_w64(e >= emax + b)) emax += b;
    return emax;
}

__device__ __forceinline__ float load_in_rt(const void* p, size_t i, int dt) {
    return dt == 0 ? load_in<0>(p, i) : dt == 1 ? load_in<1>(p, i) : load_in<2>(p, i);
}
template <int DT>
__device__ __forceinline__ void load8_in(const void* p, size_t i, float* v) {
#pragma unroll
    for (int j = 0; j < 8; ++j) v[j] = load_in<DT>(p, i + j);
}
__device__ __forceinline__ void load8_rt(const void* p, size_t i, int dt, float* v) {
    if (dt == 0) load8_in<0>(p, i, v);
    else if (dt == 1) load8_in<1>(p, i, v);
    else load8_in<2>(p, i, v);
}

// fp16 bit pattern of 2^-k (k >= 0; normal, subnormal, or 0 below 2^-24).
__device__ __forceinline__ uint32_t f16_pow2_neg(int k) {
    return k <= 14 ? (uint32_t)(15 - k) << 10 : k <= 24 ? 1u << (24 - k) : 0u;
}

constexpr float kFarBelow = -1.0e30f;  // initial maximum: exp2(score - kFarBelow) is never taken

// Byte layout of the workgroup's LDS. Loop-time areas: q' (fp32, natural
// channel order), q' as fp16 pairs in key-fragment order, and per wave the key
// steps / zero points of its tile's block (fp16 pairs, fragment order), the
// value code bytes [token][position], value steps [group][token] and the
// zero-point fragment rows [row][token]. After the loop the same bytes hold the
// four waves' output rows and their (m, l) for the merge.
template <int D, bool ROPE = false>
struct Lds {
    static constexpr int U = D / 32;
    static constexpr int VROW = D + 16;  // bytes per token row of the value tile (padded)
    static constexpr int ZROW = 40;      // halves per row of the zero-point fragment (padded)
    // q' rows padded by 4 words: the 8 lanes of a 16-byte LDS read (rows n..n+7)
    // then fall on different banks
    static constexpr int QFS = D + 4;      // floats per q' row
    static constexpr int QHS = D / 2 + 4;  // fp16 pairs per q' row
    static constexpr int QF = 0;
    static constexpr int QH = QF + 16 * QFS * 4;  // (rotary keys: no fp16 copy of q')
    static constexpr int RED = QH + (ROPE ? 0 : 16 * QHS * 4);  // 4 ints: per-wave exponent maxima
    // rotary keys, head_dim <= 128: the (cos, sin) table of the tile offsets,
    // row n + 16h = offset 8(n>>2) + 4h + (n&3) (the rows of lane n), D + 4
    // floats per row (a quarter wave's 16 rows spread over the banks)
    static constexpr bool TABLE = ROPE && D <= 128;
    static constexpr int TB = RED + 16;
    static constexpr int WAVE0 = TB + (TABLE ? 32 * (D + 4) * 4 : 0);
    static constexpr int SROW = 40;      // halves per row of the value steps (padded; cols 32.. take spare writes)
    // key step / zero-point pairs: D / 2 words plus 4 spare words for lanes without a pair.
    // Rotary keys instead: per pair slot p + p / (D/8) a float4 of the block's
    // (s_a, s_b, z_a, z_b) (RM) and the (cos, sin) of the tile's anchors (AC:
    // float2 slots p + 2 (p / (D/8)), or float4 of two anchors for head_dim 256)
    static constexpr int PPG = D / 8;
    static constexpr int ACE = D <= 128 ? 2 : 4;  // floats per anchor slot
    static constexpr int RM = 0, AC = RM + (D / 2 + 8) * 16;
    static constexpr int SP = 0, ZP = SP + D * 2 + 16,
                         VT = ROPE ? AC + (D / 2 + 16) * ACE * 4 : ZP + D * 2 + 16, ST = VT + 32 * VROW,
                         ZT = ST + U * SROW * 2;
    static constexpr int WAVE = ZT + 16 * ZROW * 2;
    static constexpr int LOOP = WAVE0 + 4 * WAVE;
    static constexpr int MO = 0, ML = 4 * 16 * D * 4;
    static constexpr int MERGE = ML + 4 * 16 * 2 * 4;
    static constexpr int BYTES = LOOP > MERGE ? LOOP : MERGE;
    static_assert(WAVE % 16 == 0 && WAVE0 % 16 == 0 && VT % 16 == 0 && ST % 16 == 0 && ZT % 16 == 0 && ZP % 16 == 0 &&
                      AC % 16 == 0,
                  "LDS alignment");
};

// One workgroup's work: split `split` of the quantized tokens of (seq, kv head
// hy / nqg, query rows 16 (hy % nqg) ..), with the layer's arguments `a`.
template <int D, int BK, int BV, bool ROPE>
__device__ __forceinline__ void gqa_body(const DecodeArgs& a, uint8_t* smem, int seq, int hy, int split) {
    constexpr int U = D / 32;                      // 32-channel units per row
    constexpr int KU = U >= 4 ? U / 4 : 1;         // key units per lane group (head_dim 64: half a unit)
    constexpr int KWL = U >= 4 ? KU * BK : BK / 2; // key words per lane and token
    constexpr int NCH = U;                         // 8-code key chunks per lane and token
    constexpr int NOT = 2 * U;                     // 16-channel output tiles
    constexpr int VRB = D * BV / 8;                // bytes of a value row
    constexpr int VUL = U / 2;                     // value units per lane (half a row)
    constexpr int VWL = VUL * BV;                  // value words per lane
    constexpr int NKP = D / 2 > 64 ? D / 128 : 1;  // key step pairs per lane per block
    constexpr int NVML = U / 2 > 1 ? U / 2 : 1;    // value metadata words per lane per tile
    constexpr int KSH = key_shift(BK), VSH = val_shift(BV);
    constexpr int KB = BV + 2, KZ = 14;
    constexpr int KLOFF = U >= 4 ? KU * BK * 4 : 2 * BK;  // byte offset between lane groups' key words
    constexpr int KALIGN = min_align(pow2_align(D * BK / 8), pow2_align(KLOFF));
    constexpr int VALIGN = pow2_align(VRB / 2);
    using KF = KeyFrag<BK>;
    using L = Lds<D, ROPE>;
    static_assert(U >= 4 || BK % 2 == 0, "head_dim 64 needs even key bits (half a unit per lane group)");
    // rotary keys: lane group g's PPG pairs, runs of PPG codes (RW words, run A
    // from word RWO of the row, run B D*BK/64 words later), the (cos, sin) of its
    // token offsets for CSH of its two token rows (head_dim 256: the first only;
    // the second row's offset, 4 more, goes into a second query anchor)
    constexpr int PPG = D / 8;
    constexpr int RW = rope_run_words<BK, PPG>();
    constexpr int CSH = D <= 128 ? 2 : 1;
    constexpr int RALIGN =
        (BK == 3 && PPG == 16) ? 4 : min_align(pow2_align(PPG * BK / 8), min_align(pow2_align(D * BK / 16), KALIGN));
    static_assert(!ROPE || D >= 128, "rotary keys on the query-group kernel: head_dim 128 or 256");

    float* qf_lds = (float*)(smem + L::QF);
    uint32_t* qh_lds = (uint32_t*)(smem + L::QH);

    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, n = lane & 15, g = lane >> 4;
    uint8_t* wbase = smem + L::WAVE0 + wave * L::WAVE;
    uint32_t* sp_lds = (uint32_t*)(wbase + L::SP);
    uint32_t* zp_lds = (uint32_t*)(wbase + L::ZP);
    uint8_t* vt_lds = wbase + L::VT;
    uint16_t* st_lds = (uint16_t*)(wbase + L::ST);  // [group][SROW]
    uint16_t* zt_lds = (uint16_t*)(wbase + L::ZT);

    const int R = a.q_heads / a.kv_heads;
    const int nqg = (R + 15) >> 4;
    const int kvh = hy / nqg, q0 = (hy - kvh * nqg) * 16;
    const int RQ = min(16, R - q0);  // query rows of this workgroup
    const int len = a.len[seq];
    // Quantized tokens [tb, te): all of them, or with a full-precision window
    // the whole key blocks inside [sinks, len - window).
    int tb, te;
    quant_range(a, len, tb, te);
    const int CW = a.chunk;
    const int wa = tb + split * CW;
    if (wa >= te) return;  // merge_kernel sees ceil((te - tb) / CW) splits
    const int wb = min(wa + CW, te);
    const SeqEntry& e = a.table[seq];
    const int lgk = a.log2_group_k, lgv = a.log2_group_v;
    const int Gk = 1 << lgk;
    const int nqk = a.win_mode ? te : (len >> lgk) << lgk;  // tokens read with quantized keys
    const int ngrp = D >> lgv;                              // value groups per token
    const int lng = __builtin_ctz(ngrp);
    const int tpg = lgv >= 4 ? 1 << (lgv - 4) : 1;          // 16-channel output tiles per value group

    // head kvh's codes and metadata inside a page (pool offsets with contiguous
    // storage); a 32-token tile lies in one page, at byte offset pb of the pool,
    // whose first token is (t0 >> psh) << psh
    const uint8_t* kc = a.codes + e.codes[0] + (size_t)kvh * e.codes_hs[0];
    const uint8_t* km = a.meta + e.meta[0] + (size_t)kvh * e.meta_hs[0];
    const uint8_t* kr = a.resid + e.resid[0] + (size_t)kvh * e.resid_hs[0];
    const uint8_t* vc = a.codes + e.codes[1] + (size_t)kvh * e.codes_hs[1];
    const uint8_t* vm = a.meta + e.meta[1] + (size_t)kvh * e.meta_hs[1];
    const int psh = e.page_shift;

    // ---- one tile of codes and metadata in registers
    uint32_t kw[2][ROPE ? 2 * RW : KWL];  // key words: token rows 8(n>>2) + 4h + (n&3), lane group g's channels
    uint32_t kmw[2 * NKP];  // key (step, zero) words of the lane's fragment pairs
    uint32_t vw[VWL];       // value words: token row lane >> 1, half lane & 1
    uint32_t vmw[NVML];     // value (step, zero) words

    // channel block (8 channels) of lane group g, chunk c
    auto cbase = [&](int c) -> int {
        if constexpr (U >= 4) return 32 * (g * KU + c / 4) + 8 * (c % 4);
        else return 32 * (g >> 1) + 16 * (g & 1) + 8 * c;
    };
    auto load_keys = [&](int t0, uint64_t pb) {
        const int wo = U >= 4 ? g * KU * BK : (g >> 1) * BK + (g & 1) * (BK / 2);
        const int ps = (t0 >> psh) << psh;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            const int t = min(t0 + 8 * (n >> 2) + 4 * h + (n & 3), nqk - 1) - ps;
            const uint32_t* row = (const uint32_t*)(kc + pb + (size_t)t * (D * BK / 8));
            if constexpr (ROPE) {
                load_n<RW, RALIGN>(row + ((PPG * BK * g) >> 5), kw[h]);
                load_n<RW, RALIGN>(row + ((PPG * BK * g) >> 5) + D * BK / 64, kw[h] + RW);
            } else {
                load_n<KWL, KALIGN>(row + wo, kw[h]);
            }
        }
    };
    auto load_kmeta = [&](int t0, uint64_t pb) {
        const int ps = (t0 >> psh) << psh;
        const uint32_t* src = (const uint32_t*)(km + pb) + (size_t)((t0 - ps) >> lgk) * D;
        if constexpr (ROPE) {  // channels p and p + D/2 of the lane's staging pairs p = lane + 64k
#pragma unroll
            for (int k = 0; k < NKP; ++k) {
                const int pp = min(lane + 64 * k, D / 2 - 1);
                kmw[2 * k] = src[pp];
                kmw[2 * k + 1] = src[pp + D / 2];
            }
            return;
        }
#pragma unroll
        for (int k = 0; k < NKP; ++k) {
            const int p = min(lane + 64 * k, D / 2 - 1), cb = (p >> 2) * 8, jj = p & 3;
            int c0 = 0, c1 = 0;
#pragma unroll
            for (int q = 0; q < 4; ++q)
                if (jj == q) c0 = KF::PERM[2 * q], c1 = KF::PERM[2 * q + 1];
            kmw[2 * k] = src[cb + c0];
            kmw[2 * k + 1] = src[cb + c1];
        }
    };
    auto load_values = [&](int t0, uint64_t pb) {
        const int ps = (t0 >> psh) << psh;
        const int t = min(t0 + (lane >> 1), wb - 1) - ps;
        load_n<VWL, VALIGN>((const uint32_t*)(vc + pb + (size_t)t * VRB + (lane & 1) * (VRB / 2)), vw);
        const uint32_t* vmp = (const uint32_t*)(vm + pb);
#pragma unroll
        for (int k = 0; k < NVML; ++k) {
            const int f = min(lane + 64 * k, 32 * ngrp - 1);
            const int tt = min(t0 + (f >> lng), wb - 1) - ps;
            vmw[k] = vmp[(size_t)tt * ngrp + (f & (ngrp - 1))];
        }
    };

    // the first tile's loads go out before the query setup, whose latency they share
    const int ntiles = (wb - wa + 31) >> 5;
    // tiles i < nqt have quantized keys (nqk and the tile starts are multiples of
    // 32); the residual-key tiles after them are handled by a loop of their own,
    // so that every load of the main loop is unconditional and the compiler's
    // wait counts stay exact
    const int nqt = nqk > wa ? min(ntiles, (nqk - wa) >> 5) : 0;
    // Lane k of pev holds the page of this wave's k-th tile of the loop below
    // (tile wave + 4k, at most 64 of them: the host keeps splits within 8192
    // tokens), so that the loop reads it with a lane read instead of a
    // dependent memory load.
    // Contiguous storage (page stride 0) skips the load, so that the first
    // tile's loads do not wait for it.
    const bool paged = e.page_bytes != 0;
    uint32_t pev = 0;
    if (wave < nqt) {
        if (paged) pev = a.pages[e.page_list + ((wa + 32 * min(wave + 4 * lane, nqt - 1)) >> psh)];
        const int t0 = wa + 32 * wave;
        const uint64_t pb = paged ? (uint64_t)(uint32_t)__builtin_amdgcn_readlane(pev, 0) * e.page_bytes : 0;
        load_values(t0, pb);
        load_kmeta(t0, pb);
        load_keys(t0, pb);
    }
    // rotary keys: per lane the frequencies of its staging pairs (and the
    // rotation by 4 positions, head_dim 256), and the (cos, sin) of its token
    // offsets u = 8(n>>2) + 4h + (n&3) for its PPG pairs from the cache's table:
    // in LDS (head_dim 128), or in registers (head_dim 256: the first row only)
    double th[NKP];
    float2 r4[NKP];
    float2 csr[L::TABLE ? 1 : CSH][L::TABLE ? 1 : PPG];
    float* tb_lds = (float*)(smem + L::TB);
    if constexpr (ROPE) {
        const float2* tab = (const float2*)a.rope_tab;
#pragma unroll
        for (int k = 0; k < NKP; ++k) {
            const int pp = min(lane + 64 * k, D / 2 - 1);
            th[k] = a.rope_theta[pp];
            r4[k] = tab[4 * (D / 2) + pp];
        }
        if constexpr (L::TABLE) {  // visible after the barrier below
            for (int i = tid; i < 32 * (D / 2); i += 256) {
                const int row = i / (D / 2), pp = i - row * (D / 2);
                const int u = 8 * ((row & 15) >> 2) + 4 * (row >> 4) + (row & 3);
                *(float2*)&tb_lds[row * (D + 4) + 2 * pp] = tab[u * (D / 2) + pp];
            }
        } else {
#pragma unroll
            for (int h = 0; h < CSH; ++h)
#pragma unroll
                for (int j = 0; j < PPG; ++j)
                    csr[h][j] = tab[(8 * (n >> 2) + 4 * h + (n & 3)) * (D / 2) + PPG * g + j];
        }
    }
    // ---- q' rows of this workgroup (rows >= RQ are 0), kept below 2^14 by
    // 2^-eqs: fp32 in natural channel order, and fp16 pairs in key-fragment order
    // (8-channel block cb: pair jj = channels cb + PERM[2jj], cb + PERM[2jj + 1])
    int eqs, eq;
    {
        const float qs = ROPE ? a.qscale : a.qscale * ((float)(1 << 8) / (float)(1 << KSH));
        const size_t qrow0 = ((size_t)seq * a.q_heads + kvh * R + q0) * D;
        float qm = 0.f;
        for (int i = tid; i < 16 * D; i += 256) {
            const int r = i / D;
            const float v = r < RQ ? load_in_rt(a.q, qrow0 + i, a.in_dtype) * qs : 0.f;
            qf_lds[r * L::QFS + (i - r * D)] = v;
            qm = fmaxf(qm, fabsf(v));
        }
        int* red = (int*)(smem + L::RED);
        const int e8w = wave_max_field<8>((int)(__float_as_uint(qm) >> 23));
        if (lane == 0) red[wave] = e8w;
        __syncthreads();
        const int e8 = max(max(red[0], red[1]), max(red[2], red[3]));  // |q'| < 2^(e8 - 126)
        eqs = max(0, e8 - 140);
        eq = e8 - eqs;
        if (eqs) {
            const float f = __builtin_amdgcn_ldexpf(1.0f, -eqs);
            for (int i = tid; i < 16 * D; i += 256) qf_lds[(i / D) * L::QFS + i % D] *= f;
            __syncthreads();
        }
        if constexpr (!ROPE) {
            for (int i = tid; i < 16 * D / 2; i += 256) {
                const int r = i / (D / 2), p = i % (D / 2), cb = (p >> 2) * 8, jj = p & 3;
                const float* qr = qf_lds + r * L::QFS + cb;
                qh_lds[r * L::QHS + p] = pk_rtz(qr[KF::PERM[2 * jj]], qr[KF::PERM[2 * jj + 1]]);
            }
        }
    }
    // constant rows of the zero-point fragment: 1.0 in row ngrp, 0 below it
    for (int i = lane; i < 16 * L::ZROW; i += 64) {
        const int r = i / L::ZROW;
        if (r >= ngrp) zt_lds[i] = r == ngrp ? (uint16_t)0x3c00u : (uint16_t)0u;
    }
    __syncthreads();

    f32x4 acc[NOT];
#pragma unroll
    for (int o = 0; o < NOT; ++o) acc[o] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 cz = {0.f, 0.f, 0.f, 0.f};  // C[query 4g+k][column n]: zero-point sums (n < ngrp), denominator (n == ngrp)
    float m = kFarBelow;              // running maximum of query n
    // the value-product exponent kb of query n (rows weight different tokens),
    // held as mb = m - kb (the weights 2^kb p = 2^(score - mb)) and zsc = 2^(KZ - kb)
    float mb = kFarBelow;
    float zsc = __builtin_amdgcn_ldexpf(1.0f, KZ - KB);
    int kb_lo = KB, kb_hi = KB;       // smallest kb of the rows < RQ, largest of all rows (wave-uniform)
    auto kb_of = [&]() { return KZ + 127 - (int)(__float_as_uint(zsc) >> 23); };

    // ---- staging of a tile's value codes (bytes), value metadata and key
    // metadata in LDS, branch-free (lanes without an item write spare slots);
    // returns the value-product exponent the tile's steps allow, and whether a
    // nonzero step is so small that 2^kb s < 2^-7 for some query row's kb (its
    // products would leave fp16's normal range, keeping few bits)
    struct TileSteps {
        int kb;     // the largest with 2^kb p s < 2^15 for every step s and p <= 1 (wave-uniform)
        bool tiny;  // wave-uniform
    };
    auto stage_values = [&]() -> TileSteps {
#pragma unroll
        for (int u = 0; u < VUL; ++u) {
            uint32_t by[8];
            unit_to_bytes<BV>(vw + u * BV, by);
            uint32_t* dst = (uint32_t*)(vt_lds + (lane >> 1) * L::VROW + ((lane & 1) * VUL + u) * 32);
            ((uint4*)dst)[0] = make_uint4(by[0], by[1], by[2], by[3]);
            ((uint4*)dst)[1] = make_uint4(by[4], by[5], by[6], by[7]);
        }
        uint32_t smx = 0, smn1 = ~0u;  // largest step, smallest nonzero step - 1 (fp16 bits: >= 0, ordered)
#pragma unroll
        for (int k = 0; k < NVML; ++k) {
            const int f = lane + 64 * k;
            const bool ok = f < 32 * ngrp;
            const int tt = f >> lng, gg = f & (ngrp - 1);
            st_lds[ok ? gg * L::SROW + tt : 32] = (uint16_t)(vmw[k] & 0xffffu);
            zt_lds[ok ? gg * L::ZROW + tt : 15 * L::ZROW + 32] = (uint16_t)(vmw[k] >> 16);
            const uint32_t sb = vmw[k] & 0x7fffu;
            smx = max(smx, ok ? sb : 0u);
            smn1 = min(smn1, ok ? sb - 1u : ~0u);
        }
        // s < 2^(e - 14) for biased fp16 exponent e: 2^kb p s < 2^15 with kb = 29 - e
        // (one ballot in the common case that no step needs kb below KB)
        const int kbt = __builtin_amdgcn_ballot_w64((int)(smx >> 10) > 29 - KB)
                            ? min(KB, 29 - wave_max_field<5>((int)(smx >> 10)))
                            : KB;
        // tiny: 0 < s < 2^et, et = -7 - min(kb_lo, kbt) >= -22; thr = fp16 bits of 2^et (inf above 2^15)
        const int et = -7 - min(kb_lo, kbt);
        const uint32_t thr = et > 15 ? 0x7c00u : et >= -14 ? (uint32_t)(et + 15) << 10 : 1u << (et + 24);
        const bool tiny = __builtin_amdgcn_ballot_w64(smn1 < thr - 1u);
        return TileSteps{kbt, tiny};
    };
    // returns fk: the key weights q' s are scaled by 2^-fk to stay in fp16 range
    auto stage_kmeta = [&]() -> int {
        uint32_t kmx = 0;
#pragma unroll
        for (int k = 0; k < NKP; ++k) {
            const int p = lane + 64 * k;
            const bool ok = p < D / 2;
            sp_lds[ok ? p : D / 2] = __builtin_amdgcn_perm(kmw[2 * k + 1], kmw[2 * k], 0x05040100u);
            zp_lds[ok ? p : D / 2] = __builtin_amdgcn_perm(kmw[2 * k + 1], kmw[2 * k], 0x07060302u);
            kmx = max(kmx, ok ? max(kmw[2 * k] & 0x7fffu, kmw[2 * k + 1] & 0x7fffu) : 0u);
        }
        // |q'| < 2^(eq - 126), s < 2^(es - 14): q' s < 2^(eq + es - 140); keep it below 2^15
        return __builtin_amdgcn_ballot_w64((int)(kmx >> 10) > 155 - eq)
                   ? max(0, eq + wave_max_field<5>((int)(kmx >> 10)) - 155)
                   : 0;
    };

    // ---- masked scores of tile t0 -> online softmax -> zero points and the value products
    auto attend = [&](float* sc, int t0, TileSteps ts) {
        if (t0 + 32 > wb) {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (t0 + 8 * g + j >= wb) sc[j] = -INFINITY;
        }
        // online softmax (exact running maximum of query n)
        float tmax = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
        tmax = col4_max(tmax);
        if (__builtin_amdgcn_ballot_w64(tmax > m)) {
            const float mnew = fmaxf(m, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);
            // row 4g + k of the accumulators belongs to query 4g + k
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float ak = __shfl(alpha, 4 * g + k);
#pragma unroll
                for (int o = 0; o < NOT; ++o) acc[o][k] *= ak;
                cz[k] *= ak;
            }
            mb = mnew - (float)kb_of();
            m = mnew;
        }
        // query n's value-product exponent: lowered when the tile's steps are
        // larger; where a step is tiny at the rows' exponents, taken from the
        // row's largest weighted step over the tile, max p s (p <= 1 against the
        // row's running maximum), up to 15 (2^kb p stays an fp16 value): a row
        // whose weight sits on tokens with small steps next to tokens with large
        // ones, or on a tile whose steps are all small, keeps the products'
        // precision. Exact rescale of the row's accumulators.
        if (ts.kb < kb_hi || ts.tiny) {
          const int kb = kb_of();
          int kbt = min(kb, ts.kb);
          if (ts.tiny) {
            float pm = 0.f;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {  // tokens 8g + 2jj, 8g + 2jj + 1: largest step over the groups
                u16x2_t sm = {};
                for (int gg = 0; gg < ngrp; ++gg)
                    sm = __builtin_elementwise_max(
                        sm, *(const u16x2_t*)&st_lds[gg * L::SROW + 8 * g + 2 * jj]);
                pm = fmaxf(pm, fmaxf(__builtin_amdgcn_exp2f(sc[2 * jj] - m) * f16_to_f32(sm[0]),
                                     __builtin_amdgcn_exp2f(sc[2 * jj + 1] - m) * f16_to_f32(sm[1])));
            }
            pm = col4_max(pm);  // over the row's 32 tokens
            // pm < 2^(e - 126) for biased fp32 exponent e: 2^kb p s < 2^15 with kb = 141 - e
            const int e = (int)(__float_as_uint(pm) >> 23);
            if (e > 0) kbt = min(15, 141 - e);  // kbt >= -113
            kb_lo = 15 - wave_max_field<8>(n < RQ ? 15 - kbt : 0);
            kb_hi = wave_max_field<8>(kbt + 114) - 114;
          } else {
            kb_lo = min(kb_lo, ts.kb);
            kb_hi = ts.kb;
          }
          if (__builtin_amdgcn_ballot_w64(kbt != kb)) {
            const float f = __builtin_amdgcn_ldexpf(1.0f, kbt - kb);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                const float fk = __shfl(f, 4 * g + k);
#pragma unroll
                for (int o = 0; o < NOT; ++o) acc[o][k] *= fk;
            }
            zsc = __builtin_amdgcn_ldexpf(1.0f, KZ - kbt);
            mb = m - (float)kbt;
          }
        }
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = exp2_for_asm(sc[j] - mb);  // mul_split's asm reads them
        uint32_t pb[4];  // 2^kb p truncated to fp16 pairs
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) pb[jj] = pk_rtz(p[2 * jj], p[2 * jj + 1]);

        // zero points and denominator
        {
            Frag ph, pl, zf;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) split2(p[2 * jj] * zsc, p[2 * jj + 1] * zsc, ph.u[jj], pl.u[jj]);
            const uint4 z4 = *(const uint4*)&zt_lds[n * L::ZROW + 8 * g];
            zf.u[0] = z4.x, zf.u[1] = z4.y, zf.u[2] = z4.z, zf.u[3] = z4.w;
            cz = mfma(ph, zf, cz);
            cz = mfma(pl, zf, cz);
        }

        // value products: output tile o = byte positions 16o..16o+15 of the value tile
        Frag sh, sl;
        const uint8_t* vrow = vt_lds + (8 * g + (n >> 1)) * L::VROW + 8 * (n & 1);
        static_for<NOT>([&](auto O) {
            constexpr int o = O;
            if ((o & (tpg - 1)) == 0) {  // first tile of a value group: P' = 2^kb p s
                const int gg = (32 * (o >> 1)) >> lgv;
                const uint4 s4 = *(const uint4*)&st_lds[gg * L::SROW + 8 * g];
                const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) mul_split(pb[jj], p[2 * jj], p[2 * jj + 1], sw[jj], sh.u[jj], sl.u[jj]);
            }
            const i32x2_t x = __builtin_amdgcn_ds_read_tr8_b64_v2i32(
                (__attribute__((address_space(3))) i32x2_t*)(vrow + 16 * o));
            const uint32_t x0 = (uint32_t)x[0], x1 = (uint32_t)x[1];  // tokens 8g..8g+3, 8g+4..8g+7
            Frag vf;
            if constexpr (VSH == 8) {
                vf.u[0] = __builtin_amdgcn_perm(x1, x0, 0x010c000cu);
                vf.u[1] = __builtin_amdgcn_perm(x1, x0, 0x030c020cu);
                vf.u[2] = __builtin_amdgcn_perm(x1, x0, 0x050c040cu);
                vf.u[3] = __builtin_amdgcn_perm(x1, x0, 0x070c060cu);
            } else {
                vf.u[0] = __builtin_amdgcn_perm(x1, x0, 0x0c010c00u) << VSH;
                vf.u[1] = __builtin_amdgcn_perm(x1, x0, 0x0c030c02u) << VSH;
                vf.u[2] = __builtin_amdgcn_perm(x1, x0, 0x0c050c04u) << VSH;
                vf.u[3] = __builtin_amdgcn_perm(x1, x0, 0x0c070c06u) << VSH;
            }
            acc[o] = mfma(sh, vf, acc[o]);
            acc[o] = mfma(sl, vf, acc[o]);
        });
    };

    // ---- rotary keys: staging of the block's metadata and the tile's anchors,
    // query and key fragments
    float* rm_lds = (float*)(wbase + L::RM);  // float4 (s_a, s_b, z_a, z_b) per pair slot
    float* ac_lds = (float*)(wbase + L::AC);  // (cos, sin) of the anchors per pair slot
    auto rslot = [](int p) { return p + p / PPG; };
    auto aslot = [](int p) { return p + (L::ACE == 2 ? 2 : 1) * (p / PPG); };
    auto stage_anchors = [&](int t0) {
#pragma unroll
        for (int k = 0; k < NKP; ++k) {
            const int pp = lane + 64 * k;
            if (pp < D / 2) {
                float c0, s0;
                rope_cs(t0, th[k], c0, s0);
                if constexpr (L::ACE == 2) {
                    *(float2*)&ac_lds[2 * aslot(pp)] = make_float2(c0, s0);
                } else {  // and the anchor t0 + 4 of the second token row
                    *(float4*)&ac_lds[4 * aslot(pp)] = make_float4(c0, s0, fmaf(c0, r4[k].x, -(s0 * r4[k].y)),
                                                                   fmaf(s0, r4[k].x, c0 * r4[k].y));
                }
            }
        }
    };
    // returns fa: the reconstructed keys (|k| <= max(|z|, |z + s (2^BK - 1)|))
    // are scaled by 2^-fa to stay below 2^14 (their rotations below 2^14.5)
    auto stage_rope = [&](int t0) -> int {
        constexpr float cmax = (float)((1 << BK) - 1);
        float sv[2 * NKP], zv[2 * NKP];
        uint32_t emx = 0;
#pragma unroll
        for (int k = 0; k < 2 * NKP; ++k) {
            sv[k] = f16_to_f32(kmw[k] & 0xffffu);
            zv[k] = f16_to_f32(kmw[k] >> 16);
            const float m = fmaxf(fabsf(zv[k]), fabsf(fmaf(sv[k], cmax, zv[k])));
            emx = max(emx, (__float_as_uint(m) >> 23) & 0xffu);
        }
        const int fa =
            __builtin_amdgcn_ballot_w64((int)emx > 140) ? max(0, wave_max_field<8>((int)emx) - 140) : 0;
        const float fs = __builtin_amdgcn_ldexpf(1.0f, -fa);
#pragma unroll
        for (int k = 0; k < NKP; ++k) {
            const int pp = lane + 64 * k;
            if (pp < D / 2) {
                const float f = __builtin_amdgcn_ldexpf(fs, 24 - rope_code_shift<BK>(pp & 3));
                *(float4*)&rm_lds[4 * rslot(pp)] =
                    make_float4(sv[2 * k] * f, sv[2 * k + 1] * f, zv[2 * k] * fs, zv[2 * k + 1] * fs);
            }
        }
        stage_anchors(t0);
        return fa;
    };
    // B of chunk pairs cb..cb+3: q' rotated back to anchor hh, fp16 hi + lo
    auto rope_b = [&](int cb, int hh, Frag& bh, Frag& bl) {
        const float4 qa4 = *(const float4*)&qf_lds[n * L::QFS + cb];
        const float4 qb4 = *(const float4*)&qf_lds[n * L::QFS + cb + D / 2];
        const float qa[4] = {qa4.x, qa4.y, qa4.z, qa4.w}, qb[4] = {qb4.x, qb4.y, qb4.z, qb4.w};
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            float c, sn;
            if constexpr (L::ACE == 2) {
                const float2 v = *(const float2*)&ac_lds[2 * aslot(cb + jj)];
                c = v.x, sn = v.y;
            } else {
                const float4 v = *(const float4*)&ac_lds[4 * aslot(cb + jj)];
                c = hh ? v.z : v.x, sn = hh ? v.w : v.y;
            }
            split2(fmaf(c, qa[jj], sn * qb[jj]), fmaf(c, qb[jj], -(sn * qa[jj])), bh.u[jj], bl.u[jj]);
        }
    };
    // A of one token row: the pair values (xa, xb) rotated by the row's offset, fp16 hi + lo
    auto rope_a = [&](const float (&xa)[4], const float (&xb)[4], int h, int c, Frag& ah, Frag& al) {
#pragma unroll
        for (int jj = 0; jj < 4; ++jj) {
            float2 r;
            if constexpr (L::TABLE) r = *(const float2*)&tb_lds[(n + 16 * h) * (D + 4) + 2 * (PPG * g + 4 * c + jj)];
            else r = csr[CSH == 2 ? h : 0][4 * c + jj];
            split2(fmaf(r.x, xa[jj], -(r.y * xb[jj])), fmaf(r.y, xa[jj], r.x * xb[jj]), ah.u[jj], al.u[jj]);
        }
    };
    // scores of a tile with quantized keys (metadata and anchors staged)
    auto rope_scores = [&](float* sc, int fa) {
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
        uint32_t ra[2][RW], rb[2][RW];  // runs A and B of the two token rows, bit-aligned
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if constexpr (BK == 3 && PPG == 16) {
                const int sh = (PPG * BK * g) & 31;
                ra[h][0] = __builtin_amdgcn_alignbit(kw[h][1], kw[h][0], sh);
                ra[h][1] = kw[h][1] >> sh;
                rb[h][0] = __builtin_amdgcn_alignbit(kw[h][3], kw[h][2], sh);
                rb[h][1] = kw[h][3] >> sh;
            } else {
#pragma unroll
                for (int k = 0; k < RW; ++k) ra[h][k] = kw[h][k], rb[h][k] = kw[h][RW + k];
            }
        }
        static_for<NCH>([&](auto C) {
            constexpr int c = C;
            const int cb = PPG * g + 4 * c;
            Frag bh[3 - CSH], bl[3 - CSH];
            rope_b(cb, 0, bh[0], bl[0]);
            if constexpr (CSH == 1) rope_b(cb, 1, bh[1], bl[1]);
            float4 m4[4];
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) m4[jj] = *(const float4*)&rm_lds[4 * rslot(cb + jj)];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                uint32_t ab[4];
                rope_chunk_codes<BK, c>(ra[h], rb[h], ab);
                float xa[4], xb[4];
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    xa[jj] = mix_lo(ab[jj], m4[jj].x, m4[jj].z);
                    xb[jj] = mix_hi(ab[jj], m4[jj].y, m4[jj].w);
                }
                Frag ah, al;
                rope_a(xa, xb, h, c, ah, al);
                const int bi = CSH == 2 ? 0 : h;
                f32x4 acc2 = h ? c1 : c0;
                acc2 = mfma(ah, bh[bi], acc2);
                acc2 = mfma(ah, bl[bi], acc2);
                acc2 = mfma(al, bh[bi], acc2);
                if (h) c1 = acc2;
                else c0 = acc2;
            }
        });
        const float cs = __builtin_amdgcn_ldexpf(1.0f, eqs + fa);
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            sc[k] = c0[k] * cs;
            sc[4 + k] = c1[k] * cs;
        }
    };

    // ---- tiles with quantized keys: the next tile's words are requested as
    // soon as this tile's are consumed (the last tile re-requests itself)
    for (int i = wave, k = 0; i < nqt; i += 4, ++k) {
        const int t0 = wa + 32 * i;
        const bool more = i + 4 < nqt;
        const int tn = wa + 32 * (more ? i + 4 : i);
        const uint64_t pbn =
            paged ? (uint64_t)(uint32_t)__builtin_amdgcn_readlane(pev, more ? k + 1 : k) * e.page_bytes : 0;
        const TileSteps kb_tile = stage_values();
        int fk;
        if constexpr (ROPE) fk = stage_rope(t0);
        else fk = stage_kmeta();
        __builtin_amdgcn_sched_barrier(0);
        load_values(tn, pbn);
        load_kmeta(tn, pbn);
        __builtin_amdgcn_sched_barrier(0);  // the requests go out before the arithmetic
        wave_lds_sync();

        // key scores: sc[j] for query n, token t0 + 8g + j
        float sc[8];
        if constexpr (ROPE) {
            rope_scores(sc, fk);
            __builtin_amdgcn_sched_barrier(0);
            load_keys(tn, pbn);
            __builtin_amdgcn_sched_barrier(0);
        } else {
            f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
            float bz = 0.f;
            const uint32_t fpair = f16_pow2_neg(fk) * 0x10001u;
            static_for<NCH>([&](auto C) {
                constexpr int c = C;
                const int cb = cbase(c);
                const float4 qa = *(const float4*)&qf_lds[n * L::QFS + cb];
                const float4 qb = *(const float4*)&qf_lds[n * L::QFS + cb + 4];
                const float qv[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
                const uint4 qh4 = *(const uint4*)&qh_lds[n * L::QHS + cb / 2];
                uint4 sp4 = *(const uint4*)&sp_lds[cb / 2];
                const uint4 zp4 = *(const uint4*)&zp_lds[cb / 2];
                if (fk) {
                    sp4.x = pk_mul(sp4.x, fpair), sp4.y = pk_mul(sp4.y, fpair);
                    sp4.z = pk_mul(sp4.z, fpair), sp4.w = pk_mul(sp4.w, fpair);
                }
                const uint32_t qh[4] = {qh4.x, qh4.y, qh4.z, qh4.w};
                const uint32_t sp[4] = {sp4.x, sp4.y, sp4.z, sp4.w};
                const uint32_t zp[4] = {zp4.x, zp4.y, zp4.z, zp4.w};
                Frag bh, bl;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) {
                    const float qx = qv[KF::PERM[2 * jj]], qy = qv[KF::PERM[2 * jj + 1]];
                    mul_split(qh[jj], qx, qy, sp[jj], bh.u[jj], bl.u[jj]);
                    bz = mix_lo(zp[jj], qx, bz);
                    bz = mix_hi(zp[jj], qy, bz);
                }
                Frag a0f, a1f;
                KF::template get<c>(kw[0], a0f);
                KF::template get<c>(kw[1], a1f);
                c0 = mfma(a0f, bh, c0);
                c0 = mfma(a0f, bl, c0);
                c1 = mfma(a1f, bh, c1);
                c1 = mfma(a1f, bl, c1);
            });
            __builtin_amdgcn_sched_barrier(0);
            load_keys(tn, pbn);
            __builtin_amdgcn_sched_barrier(0);
            const float bias = col4_sum(bz) * __builtin_amdgcn_ldexpf(1.0f, KSH - 8 + eqs);
            const float cs = __builtin_amdgcn_ldexpf(1.0f, 16 + fk + eqs);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sc[k] = fmaf(c0[k], cs, bias);
                sc[4 + k] = fmaf(c1[k], cs, bias);
            }
        }
        attend(sc, t0, kb_tile);
        wave_lds_sync();  // the next stage rewrites this wave's LDS areas
    }

    // ---- tiles whose keys are still in the residual (the last, incomplete key
    // block: at most one block per sequence), loaded as they come
    for (int i = wave; i < ntiles; i += 4) {
        if (i < nqt) continue;
        const int t0 = wa + 32 * i;
        load_values(t0, (uint64_t)a.pages[e.page_list + (t0 >> psh)] * e.page_bytes);
        const TileSteps kb_tile = stage_values();
        if constexpr (ROPE) stage_anchors(t0);
        wave_lds_sync();
        float sc[8];
        if constexpr (ROPE) {  // input rows rotated by their offsets, q' rotated back to the tile's anchors
            f32x4 c[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            static_for<NCH>([&](auto C) {
                constexpr int cc = C;
                const int cb = PPG * g + 4 * cc;
                Frag bh[3 - CSH], bl[3 - CSH];
                rope_b(cb, 0, bh[0], bl[0]);
                if constexpr (CSH == 1) rope_b(cb, 1, bh[1], bl[1]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int t = min(t0 + 8 * (n >> 2) + 4 * h + (n & 3), wb - 1);
                    const size_t base = (size_t)(t & (Gk - 1)) * D + cb;
                    float xa[4], xb[4];
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) {
                        xa[jj] = load_in_rt(kr, base + jj, a.in_dtype);
                        xb[jj] = load_in_rt(kr, base + D / 2 + jj, a.in_dtype);
                    }
                    Frag ah, al;
                    rope_a(xa, xb, h, cc, ah, al);
                    const int bi = CSH == 2 ? 0 : h;
                    c[h] = mfma(ah, bh[bi], c[h]);
                    c[h] = mfma(ah, bl[bi], c[h]);
                    c[h] = mfma(al, bh[bi], c[h]);
                }
            });
            const float cs = __builtin_amdgcn_ldexpf(1.0f, eqs);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sc[k] = c[0][k] * cs;
                sc[4 + k] = c[1][k] * cs;
            }
        } else {
            // keys and queries both as fp16 hi + lo (three MFMAs)
            f32x4 c[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
            static_for<NCH>([&](auto C) {
                constexpr int cc = C;
                const int cb = cbase(cc);
                const float4 qa = *(const float4*)&qf_lds[n * L::QFS + cb];
                const float4 qb = *(const float4*)&qf_lds[n * L::QFS + cb + 4];
                Frag bh, bl;
                split2(qa.x, qa.y, bh.u[0], bl.u[0]);
                split2(qa.z, qa.w, bh.u[1], bl.u[1]);
                split2(qb.x, qb.y, bh.u[2], bl.u[2]);
                split2(qb.z, qb.w, bh.u[3], bl.u[3]);
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    const int t = min(t0 + 8 * (n >> 2) + 4 * h + (n & 3), wb - 1);
                    float kv[8];
                    load8_rt(kr, (size_t)(t & (Gk - 1)) * D + cb, a.in_dtype, kv);
                    Frag ah, al;
#pragma unroll
                    for (int jj = 0; jj < 4; ++jj) split2(kv[2 * jj], kv[2 * jj + 1], ah.u[jj], al.u[jj]);
                    c[h] = mfma(ah, bh, c[h]);
                    c[h] = mfma(ah, bl, c[h]);
                    c[h] = mfma(al, bh, c[h]);
                }
            });
            const float cs = __builtin_amdgcn_ldexpf(1.0f, KSH - 8 + eqs);
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                sc[k] = c[0][k] * cs;
                sc[4 + k] = c[1][k] * cs;
            }
        }
        attend(sc, t0, kb_tile);
        wave_lds_sync();
    }

    // ---- merge the four waves (fixed order) and write this split's partial (m, l, o)
    float* mo = (float*)(smem + L::MO);  // [wave][row][channel]
    float* ml = (float*)(smem + L::ML);  // [wave][row][m, l]
    wg_lds_barrier();                    // every wave is done with the loop areas
    {
        const float oscale = zsc * (float)(1 << (24 - VSH - KZ));  // 2^(24 - kb - VSH) of query n
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int r = 4 * g + k;
            const float osk = __shfl(oscale, r);
#pragma unroll
            for (int o = 0; o < NOT; ++o) {
                const int gg = (32 * (o >> 1)) >> lgv;
                const float zs = __shfl(cz[k], 16 * g + gg) * (1.0f / (float)(1 << KZ));
                const int ch = 32 * (o >> 1) + val_chan<BV>(16 * (o & 1) + n);
                mo[(wave * 16 + r) * D + ch] = fmaf(acc[o][k], osk, zs);
            }
            if (n == ngrp) ml[(wave * 16 + r) * 2 + 1] = cz[k] * (1.0f / (float)(1 << KZ));
        }
        if (g == 0) ml[(wave * 16 + n) * 2] = m;
    }
    wg_lds_barrier();
    for (int idx = tid; idx < RQ * D; idx += 256) {
        const int r = idx / D, ch = idx - r * D;
        float M = ml[r * 2];
#pragma unroll
        for (int w = 1; w < 4; ++w) M = fmaxf(M, ml[(w * 16 + r) * 2]);
        float o = 0.f, l = 0.f;
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            const float sw = __builtin_amdgcn_exp2f(ml[(w * 16 + r) * 2] - M);
            o = fmaf(mo[(w * 16 + r) * D + ch], sw, o);
            l = fmaf(ml[(w * 16 + r) * 2 + 1], sw, l);
        }
        const size_t slot = ((size_t)seq * a.q_heads + kvh * R + q0 + r) * a.max_chunks + split;
        a.ws_o[slot * D + ch] = o;
        if (ch == 0) {
            a.ws_ml[slot * 2 + 0] = M;
            a.ws_ml[slot * 2 + 1] = l;
        }
    }
}

// Keys cached before the rotary embedding: the instantiations of the objects
// built with KVQ_GQA_ROPE (fewer waves per SIMD: the rotated fragments, and at
// head_dim 256 the lane's (cos, sin), need the registers). The split choice
// assumes these bounds (gqa_resident_per_cu).
#if KVQ_GQA_ROPE
constexpr bool kRope = true;
#if KVQ_GQA_HEAD_DIM > 128  // head_dim 256 keeps its (cos, sin) in registers: one wave per SIMD
#define KVQ_GQA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(1, 1)))
#else
#define KVQ_GQA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(2, 2)))
#endif
#else
constexpr bool kRope = false;
#if KVQ_GQA_HEAD_DIM > 128  // the LDS of a head_dim 256 workgroup leaves room for two per compute unit
#define KVQ_GQA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(2, 2)))
#else
#define KVQ_GQA_OCCUPANCY __attribute__((amdgpu_waves_per_eu(3, 3)))
#endif
#endif

// One launch per (bits_k, bits_v) pair: grid = (split, kv head x query group,
// the pair's sequences x layers).
template <int D, int BK, int BV, bool ROPE>
__global__ __launch_bounds__(256) KVQ_GQA_OCCUPANCY void decode_gqa_kernel(DecodeArgs a0) {
    __shared__ __align__(16) uint8_t smem[Lds<D, ROPE>::BYTES];
    int z = blockIdx.z;
    const DecodeArgs a = layer_args(a0, z, gridDim.z / a0.n_layers);
    gqa_body<D, BK, BV, ROPE>(a, smem, a.seq_list ? a.seq_list[z] : z, blockIdx.y, blockIdx.x);
}

template <int D, int BK, bool ROPE>
__device__ __forceinline__ void gqa_list_bv(int bv, const DecodeArgs& a, uint8_t* smem, int seq, int hy, int split) {
    switch (bv) {
        case 2: gqa_body<D, BK, 2, ROPE>(a, smem, seq, hy, split); break;
        case 3: gqa_body<D, BK, 3, ROPE>(a, smem, seq, hy, split); break;
        case 4: gqa_body<D, BK, 4, ROPE>(a, smem, seq, hy, split); break;
        case 6: gqa_body<D, BK, 6, ROPE>(a, smem, seq, hy, split); break;
        default: gqa_body<D, BK, 8, ROPE>(a, smem, seq, hy, split); break;
    }
}

// Every bit pair of the call in one launch: workgroup f takes the f-th active
// (layer, seq, split, kv head x query group) item of a list ordered by bit
// pair, found by binary search over the list's per-(layer, seq) starts.
template <int D, bool ROPE>
__global__ __launch_bounds__(256) KVQ_GQA_OCCUPANCY void decode_gqa_list_kernel(DecodeArgs a0, GqaList list) {
    __shared__ __align__(16) uint8_t smem[Lds<D, ROPE>::BYTES];
    const int f = blockIdx.x;
    int lo = 0, hi = list.count - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (list.start[mid] <= f) lo = mid;
        else hi = mid - 1;
    }
    const int seq = list.seq[lo];
    int z = list.layer[lo] * a0.num_seqs + seq;
    const DecodeArgs a = layer_args(a0, z, a0.num_seqs);
    const int R = a.q_heads / a.kv_heads;
    const int nh = a.kv_heads * ((R + 15) >> 4);
    const int r = f - list.start[lo];
    const SeqEntry& e = a.table[seq];
    const int bk = e.bits[0], bv = e.bits[1];
    switch (bk) {
        case 2: gqa_list_bv<D, 2, ROPE>(bv, a, smem, seq, r % nh, r / nh); break;
        case 3:
            if constexpr (D >= 128) gqa_list_bv<D, 3, ROPE>(bv, a, smem, seq, r % nh, r / nh);
            break;
        case 4: gqa_list_bv<D, 4, ROPE>(bv, a, smem, seq, r % nh, r / nh); break;
        case 6: gqa_list_bv<D, 6, ROPE>(bv, a, smem, seq, r % nh, r / nh); break;
        default: gqa_list_bv<D, 8, ROPE>(bv, a, smem, seq, r % nh, r / nh); break;
    }
}

template <int D, int BK>
hipError_t gqa_bv(const DecodeArgs& a, int bv, dim3 grid, hipStream_t s) {
    const dim3 block(256);
    switch (bv) {
        case 2: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 2, kRope>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 3, kRope>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 4, kRope>), grid, block, 0, s, a); break;
        case 6: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 6, kRope>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 8, kRope>), grid, block, 0, s, a); break;
    }
    return hipGetLastError();
}

template <int D>
hipError_t gqa_bk(const DecodeArgs& a, int bk, int bv, dim3 grid, hipStream_t s) {
    switch (bk) {
        case 2: return gqa_bv<D, 2>(a, bv, grid, s);
        case 3:
            if constexpr (D >= 128) return gqa_bv<D, 3>(a, bv, grid, s);
            else return hipErrorInvalidValue;
        case 4: return gqa_bv<D, 4>(a, bv, grid, s);
        case 6: return gqa_bv<D, 6>(a, bv, grid, s);
        default: return gqa_bv<D, 8>(a, bv, grid, s);
    }
}

}  // namespace

// Compiled once per head_dim (KVQ_GQA_HEAD_DIM = 64, 128, 256), and with
// KVQ_GQA_ROPE = 1 for head_dim 128 and 256 (the rotary instantiations).
#define KVQ_GCAT2(a, b) a##b
#define KVQ_GCAT(a, b) KVQ_GCAT2(a, b)
#if KVQ_GQA_ROPE
#define KVQ_GQA_LIST KVQ_GCAT(launch_decode_gqa_rope_list_d, KVQ_GQA_HEAD_DIM)
#define KVQ_GQA_LAUNCH KVQ_GCAT(launch_decode_gqa_rope_d, KVQ_GQA_HEAD_DIM)
#else
#define KVQ_GQA_LIST KVQ_GCAT(launch_decode_gqa_list_d, KVQ_GQA_HEAD_DIM)
#define KVQ_GQA_LAUNCH KVQ_GCAT(launch_decode_gqa_d, KVQ_GQA_HEAD_DIM)
#endif
hipError_t KVQ_GQA_LIST(const DecodeArgs& a, const GqaList& list, int items, hipStream_t s) {
    hipLaunchKernelGGL((decode_gqa_list_kernel<KVQ_GQA_HEAD_DIM, kRope>), dim3(items), dim3(256), 0, s, a, list);
    return hipGetLastError();
}

hipError_t KVQ_GQA_LAUNCH(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s) {
    // x: the quantized splits only (the workspace's full-precision slots have no
    // workgroups here: empty ones would leave the busy ones on a few XCDs);
    // y: kv heads x groups of 16 query heads
    const int R = a.q_heads / a.kv_heads;
    dim3 grid(a.max_chunks - a.win_splits, a.kv_heads * ((R + 15) / 16), nseqs * a.n_layers);
    return gqa_bk<KVQ_GQA_HEAD_DIM>(a, bits_k, bits_v, grid, s);
}

}  // namespace kvq
