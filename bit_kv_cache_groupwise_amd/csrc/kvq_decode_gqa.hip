// Decode attention for query groups (q_heads / kv_heads = R in 2..16): the R
// queries that share a kv head turn the decode step into a small dense
// contraction, so both products run on MFMA (v_mfma_f32_16x16x32_f16) with the
// packed codes as exact fp16 operands. Keys on the channel axis, values on the
// token axis.
//
// Sources, by page title and section:
//   [N] nalar.dev, "Kuantisasi KV cache untuk mengurangi memory inferensi
//       long-context", "Kuantisasi dapat memindahkan pekerjaan ke decode path"
//   [N] same page, "Ukuran cache bertambah mengikuti token, layer, dan KV head"
//       (grouped-query attention shares kv heads among query heads)
//
// Work decomposition: workgroup = (split of the token axis, kv head, seq); its
// waves share every 32-token tile, wave w owning 64 of the head's channels
// (128 for 3-bit keys). Per tile a wave computes
//   partial scores^T[t][r] = 2^16 * sum_c A[t][c] B[c][r] + bias[r] over its channels,
//     A = key codes of token t as fp16 values (code << sh) * 2^-24, unpacked
//         from the lane's own row words (exact),
//     B = q'_rc * s_c in fp16 hi + lo parts (two MFMAs), where q' carries the
//         2^(8-sh) that undoes the code shift,
//     bias[r] = sum_c q_rc z_c on the VALU;
//   the waves' partial scores are summed through LDS (one barrier per tile);
//   O[r][c]  += 2^(24-kb-sh) * sum_t (2^kb p_rt s_t,g(c))[hi + lo] V[t][c],
//     kb = the wave's running value-product exponent (at most BV + 2, lowered
//     when a tile's largest value step would push 2^kb p s past 2^15),
//     V = value codes as fp16 values (code << sh) * 2^-24, from an LDS byte tile;
//   Z[r][g]  += 2^-KZ * sum_t (2^KZ p_rt)[hi + lo] * (z_t,g | 1),
//     one MFMA against a [token][group] fragment of zero points whose column
//     after the last group is 1, so it also yields the softmax denominator.
// The score layout (lane: 1 query x 8 consecutive tokens) is the operand layout
// the value products need for P, so softmax weights never leave registers.
//
// Pipeline: the next tile's codes and metadata are loaded into registers as
// soon as the current ones are consumed (value words after they are staged in
// LDS, key words after the score MFMAs), so every wave keeps one tile in
// flight while it computes the current one.
//
// Softmax: online in the log2 domain with the exact running maximum, so
// weights are <= 1; they enter the fp16 operands pre-scaled by powers of two
// (2^(BV+2) for p * s, 2^14 for the zero-point / denominator product) so that
// small weights keep full fp16 precision. Splits are merged by merge_kernel.
#include <utility>

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

using namespace dev;

typedef _Float16 half8_t __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

union Frag {
    half8_t h;
    uint32_t u[4];
};

__device__ __forceinline__ f32x4 mfma(const Frag& a, const Frag& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(a.h, b.h, c, 0, 0, 0);
}

template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
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

// Integer codes enter the MFMAs as fp16 values code * 2^(sh-24): subnormals,
// or normals of exponent 1, where the value is still (code << sh) * 2^-24.
// The MFMA's sum of products loses low bits of products whose subnormal
// operand uses only the bottom of the mantissa, so every code is shifted until
// its top bit reaches bit 9 or 10 (code << sh < 2048): sh = code_shift(B).
__host__ __device__ constexpr int code_shift(int B) { return B == 2 ? 9 : B == 3 ? 8 : B == 4 ? 7 : B == 6 ? 5 : 3; }

// Key-code fragments: chunk k of a lane's channel range (8 channels) as 8 fp16
// halves. Half j of the fragment holds channel 8k + PERM[j] of the range as the
// integer code << code_shift(B).
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

// Code j (0..31) of one packed 32-channel unit (little-endian bitstream).
template <int B, int J>
__device__ __forceinline__ uint32_t unit_code(const uint32_t* w) {
    constexpr int pos = J * B, wi = pos >> 5, sh = pos & 31;
    if constexpr (sh + B <= 32) return (w[wi] >> sh) & ((1u << B) - 1u);
    else return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << B) - 1u);
}

// 3- and 6-bit codes straddle words: one bit-field extract per code.
template <int B>
struct KeyFragStraddle {
    static constexpr int PERM[8] = {0, 1, 2, 3, 4, 5, 6, 7};
    static constexpr int SH = code_shift(B);
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

// N consecutive words from p, whose byte address is a multiple of ALIGN. Plain
// loads, not the non-temporal streaming ones: the waves of a workgroup read
// different channel slices of the same cache lines, and the hint made those
// lines miss for the later waves (~20% slower on a 262k-token query group).
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
template <int N>
__device__ __forceinline__ void store_lds_n(uint32_t* p, const uint32_t* w) {
    if constexpr (N % 4 == 0) {
#pragma unroll
        for (int k = 0; k < N / 4; ++k) ((uint4*)p)[k] = make_uint4(w[4 * k], w[4 * k + 1], w[4 * k + 2], w[4 * k + 3]);
    } else if constexpr (N % 2 == 0) {
#pragma unroll
        for (int k = 0; k < N / 2; ++k) ((uint2*)p)[k] = make_uint2(w[2 * k], w[2 * k + 1]);
    } else {
        p[0] = w[0];
    }
}

constexpr int pow2_align(int bytes) { return (bytes & 15) == 0 ? 16 : (bytes & 7) == 0 ? 8 : (bytes & 3) == 0 ? 4 : 1; }

// Sums and maxima over the 4 lanes that share l % 16 (lanes l, l^16, l^32, l^48),
// with the row-swap permutes (no LDS round trip): after permlane16_swap(v, v)
// the two results hold rows (0,0,2,2) and (1,1,3,3); after permlane32_swap(v, v)
// they hold halves (lo, lo) and (hi, hi).
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

__device__ __forceinline__ void wave_lds_sync() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
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

constexpr float kTwo16 = 65536.0f;
constexpr float kTwo24 = 16777216.0f;
constexpr float kFarBelow = -1.0e30f;  // initial reference maximum: exp2(score - kFarBelow) never taken

// Channels per wave: the workgroup's waves share each tile, wave w taking
// channels [w*DW, (w+1)*DW) of the head. A lane group of a wave must own whole
// key words, so 3-bit keys take 128 channels per wave.
template <int BK>
constexpr int wave_channels() { return BK == 3 ? 128 : 64; }

__device__ __forceinline__ void wg_lds_barrier() {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    __builtin_amdgcn_s_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Three waves per SIMD for 64-channel waves (registers capped at 168, no
// spills); 128-channel waves need more and run two.
template <int D, int BK, int BV>
__global__ __launch_bounds__(D / wave_channels<BK>() * 64)
__attribute__((amdgpu_waves_per_eu(BK == 3 ? 2 : 3, BK == 3 ? 2 : 3))) void decode_gqa_kernel(DecodeArgs a0) {
    int z = blockIdx.z;
    const DecodeArgs a = layer_args(a0, z, gridDim.z / a0.n_layers);
    constexpr int DW = wave_channels<BK>();  // channels of this wave
    constexpr int NWV = D / DW;               // waves per workgroup (they share every tile)
    constexpr int NT = 64 * NWV;
    constexpr int DQ = DW / 4;                // key channels of one lane group (lg)
    constexpr int NCH = DQ / 8;               // 8-channel MFMA chunks per lane group
    constexpr int NSUB = DW / 16;             // 16-column output tiles of the wave
    constexpr int KWL = DQ * BK / 32;         // key words of a lane per token
    constexpr int VROW = DW + 8;              // bytes per token row of the wave's value tile
    constexpr int UPW = DW / 32;              // value units of the wave per token
    constexpr int UPL = UPW / 2;              // value units per lane per tile (32 tokens)
    constexpr int NVML = DW / 64;             // value metadata words per lane per tile
    constexpr int ZROW = 40;                  // halves per row of the zero-point tile (padded)
    constexpr int KALIGN = pow2_align(D * BK / 8) < pow2_align(KWL * 4) ? pow2_align(D * BK / 8) : pow2_align(KWL * 4);
    constexpr int VALIGN = pow2_align(D * BV / 8) < pow2_align(BV * 4) ? pow2_align(D * BV / 8) : pow2_align(BV * 4);
    constexpr int KSH = code_shift(BK), VSH = code_shift(BV);
    // Softmax weight scales (p <= 1): 2^kb p * s with kb <= KB = BV + 2 keeps
    // small weights normal in fp16; kb drops below KB where a tile's value
    // steps are large (running_value_exponent), so that 2^kb p s < 2^15;
    // 2^KZ p <= 16384.
    constexpr int KB = BV + 2, KZ = 14;
    constexpr int XS = 2 * NWV * 64 * 8 > NWV * 16 * DW ? 2 * NWV * 64 * 8 : NWV * 16 * DW;
    using KF = KeyFrag<BK>;
    static_assert(KWL * 32 == DQ * BK, "lane key range must be whole words");
    static_assert(UPL >= 1 && NVML >= 1, "wave tile shape");

    // Key pairs follow the fragment order: dword 4w + jj of a wave row holds
    // channels 8w + PERM[2jj] (low half) and 8w + PERM[2jj+1] (high half).
    __shared__ __align__(16) float xbuf[XS];                   // partial scores [2][NWV][64][8]; output staging
    __shared__ __align__(16) uint32_t sp_lds[NWV][DW / 2];     // key scales of the tile's block, fp16 pairs
    __shared__ __align__(16) uint32_t zp_lds[NWV][DW / 2];     // key zero points, fp16 pairs
    __shared__ __align__(16) uint8_t vt_lds[NWV][32 * VROW];  // value codes of the tile, one byte each
    __shared__ __align__(16) uint16_t st_lds[NWV][4][32];     // value scales [group][token]
    __shared__ __align__(16) uint16_t zt_lds[NWV][16][ZROW];  // value zero points [group][token]; row G = 1.0

    const int seq = a.seq_list ? a.seq_list[z] : z;
    const int kvh = blockIdx.y, split = blockIdx.x;
    const int len = a.len[seq];
    // Quantized tokens [tb, te): all of them, or with a full-precision window
    // the whole key blocks inside [sinks, len - window).
    int tb, te;
    quant_range(a, len, tb, te);
    const int CW = a.chunk;
    const int wa = tb + split * CW;
    if (wa >= te) return;  // merge_kernel sees ceil((te - tb) / CW) splits
    const int wb = min(wa + CW, te);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ln = lane & 15, lg = lane >> 4;
    const int cw0 = wave * DW;  // first channel of this wave
    const int R = a.q_heads / a.kv_heads;
    const SeqEntry& e = a.table[seq];
    const int lgk = a.log2_group_k, lgv = a.log2_group_v;
    const int Gk = 1 << lgk;
    const int nqk = a.win_mode ? te : (len >> lgk) << lgk;  // tokens read with quantized keys
    const int qend = min(wb, nqk);
    const int vgpr = D >> lgv;            // value groups per token
    const int g0 = cw0 >> lgv;            // first value group of this wave
    const int ngw = lgv <= 5 + __builtin_ctz(UPW) ? DW >> lgv : 1;  // value groups of this wave
    const int lng = __builtin_ctz(ngw);
    const int bpg = lgv - 5;              // log2 of 32-channel blocks per value group

    const uint8_t* kc = a.codes + e.codes[0] + (size_t)kvh * e.codes_hs[0];
    const uint32_t* km = (const uint32_t*)(a.meta + e.meta[0] + (size_t)kvh * e.meta_hs[0]);
    const uint8_t* kr = a.resid + e.resid[0] + (size_t)kvh * e.resid_hs[0];
    const uint8_t* vc = a.codes + e.codes[1] + (size_t)kvh * e.codes_hs[1];
    const uint32_t* vm = (const uint32_t*)(a.meta + e.meta[1] + (size_t)kvh * e.meta_hs[1]);

    // ---- query ln of this kv head, channels cw0 + lg*DQ + [0, DQ), in registers:
    // q' = q * scale * 2^(8 - KSH) and its fp16 pairs in fragment order
    float qf[DQ];
    uint32_t qh[DQ / 2];
    {
        const size_t qrow = ((size_t)seq * a.q_heads + kvh * R + min(ln, R - 1)) * D + cw0 + lg * DQ;
#pragma unroll
        for (int k = 0; k < NCH; ++k) load8_rt(a.q, qrow + 8 * k, a.in_dtype, qf + 8 * k);
#pragma unroll
        for (int j = 0; j < DQ; ++j) qf[j] = ln < R ? qf[j] * a.qscale * ((float)(1 << 8) / (float)(1 << KSH)) : 0.f;
#pragma unroll
        for (int k = 0; k < NCH; ++k)
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                qh[4 * k + jj] = pk_rtz(qf[8 * k + KF::PERM[2 * jj]], qf[8 * k + KF::PERM[2 * jj + 1]]);
    }
    // constant rows of the zero-point fragment: 1.0 in row ngw, 0 above it
    for (int i = lane; i < 16 * 32; i += 64) {
        const int g = i >> 5;
        if (g >= ngw) zt_lds[wave][g][i & 31] = g == ngw ? (uint16_t)0x3c00u : (uint16_t)0u;
    }

    f32x4 acc[NSUB];
#pragma unroll
    for (int n = 0; n < NSUB; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 cz = {0.f, 0.f, 0.f, 0.f};  // C[query 4lg+i][col ln]: zero-point sums (ln < ngw), denominator (ln == ngw)
    float m = kFarBelow;              // reference maximum of query ln (the same in every wave)
    int kb = KB;                      // value-product exponent (wave-uniform, never rises)
    int kb_tile = KB;                 // the exponent the staged tile's value steps allow

    // ---- prefetch registers: two sets, so the tiles two ahead are in flight
    struct Pref {
        uint32_t kw[2][KWL];   // key words of token rows 8(ln>>2) + 4s + (ln&3), lane group lg
        uint32_t kmw[2];       // the two key metadata words of this lane's fragment pair
        uint32_t vw[UPL][BV];  // value units of the wave
        uint32_t vmw[NVML];    // value metadata words
    };
    Pref pf[2];

    auto load_keys = [&](Pref& P, int t0) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int t = min(t0 + 8 * (ln >> 2) + 4 * s + (ln & 3), nqk - 1);
            load_n<KWL, KALIGN>((const uint32_t*)(kc + (size_t)t * (D * BK / 8) + (cw0 + lg * DQ) * BK / 8), P.kw[s]);
        }
    };
    // Lane -> fragment pair (window kw8, pair kjj) of the wave's key channels.
    const int kpair = lane % (DW / 2), kw8 = kpair >> 2, kjj = kpair & 3;
    auto load_kmeta = [&](Pref& P, int t0) {
        const uint32_t* src = km + (size_t)(t0 >> lgk) * D + cw0 + 8 * kw8;
        int c0 = 0, c1 = 0;
#pragma unroll
        for (int jj = 0; jj < 4; ++jj)
            if (kjj == jj) c0 = KF::PERM[2 * jj], c1 = KF::PERM[2 * jj + 1];
        P.kmw[0] = src[c0];
        P.kmw[1] = src[c1];
    };
    auto load_values = [&](Pref& P, int t0) {
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int f = lane + 64 * u;
            const int t = min(t0 + f / UPW, wb - 1);
            load_n<BV, VALIGN>((const uint32_t*)(vc + (size_t)t * (D * BV / 8) + (cw0 / 32 + f % UPW) * BV * 4), P.vw[u]);
        }
        // a fixed count of loads (clamped indices), so the compiler's wait counts
        // never have to assume a load was skipped
#pragma unroll
        for (int u = 0; u < NVML; ++u) {
            const int f = min(lane + 64 * u, 32 * ngw - 1);
            const int t = min(t0 + (f >> lng), wb - 1);
            P.vmw[u] = vm[(size_t)t * vgpr + g0 + (f & (ngw - 1))];
        }
    };
    // Stage value bytes, value scales / zero points and key metadata of the tile in LDS.
    auto stage = [&](Pref& P, bool with_keys) {
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int f = lane + 64 * u;
            uint32_t by[8];
            unit_to_bytes<BV>(P.vw[u], by);
            uint32_t* dst = (uint32_t*)&vt_lds[wave][(f / UPW) * VROW + (f % UPW) * 32];
#pragma unroll
            for (int k = 0; k < 4; ++k) ((uint2*)dst)[k] = make_uint2(by[2 * k], by[2 * k + 1]);
        }
        uint32_t smx = 0;  // largest fp16 value step of the wave's tile (steps are >= 0: bit order = value order)
#pragma unroll
        for (int u = 0; u < NVML; ++u) {
            const int f = lane + 64 * u;
            if (f < 32 * ngw) {
                const int tt = f >> lng, g = f & (ngw - 1);
                st_lds[wave][g][tt] = (uint16_t)(P.vmw[u] & 0xffffu);
                zt_lds[wave][g][tt] = (uint16_t)(P.vmw[u] >> 16);
                smx = max(smx, P.vmw[u] & 0x7fffu);
            }
        }
        // the wave's largest biased exponent e (a scalar: binary search over ballots);
        // s < 2^(e - 14), so 2^kb p s < 2^15 with kb = 29 - e
        const int el = (int)(smx >> 10);
        int emax = 0;
#pragma unroll
        for (int b = 16; b; b >>= 1)
            if (__builtin_amdgcn_ballot_w64(el >= emax + b)) emax += b;
        kb_tile = min(KB, 29 - emax);
        if (with_keys && lane < DW / 2) {
            sp_lds[wave][kpair] = __builtin_amdgcn_perm(P.kmw[1], P.kmw[0], 0x05040100u);
            zp_lds[wave][kpair] = __builtin_amdgcn_perm(P.kmw[1], P.kmw[0], 0x07060302u);
        }
    };

    // Partial key scores over this wave's channels of a quantized tile:
    // sc[j] for query ln, token t0 + 8lg + j.
    auto key_scores_quant = [&](const Pref& P, float* sc) {
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
        float bz = 0.f;
        uint4 spc = *(const uint4*)&sp_lds[wave][4 * (lg * NCH)];
        uint4 zpc = *(const uint4*)&zp_lds[wave][4 * (lg * NCH)];
        static_for<NCH>([&](auto K) {
            constexpr int k = K;
            uint4 spn, zpn;
            if constexpr (k + 1 < NCH) {  // one chunk of LDS reads in flight
                spn = *(const uint4*)&sp_lds[wave][4 * (lg * NCH + k + 1)];
                zpn = *(const uint4*)&zp_lds[wave][4 * (lg * NCH + k + 1)];
            }
            const uint32_t sp[4] = {spc.x, spc.y, spc.z, spc.w};
            const uint32_t zp[4] = {zpc.x, zpc.y, zpc.z, zpc.w};
            Frag bh, bl;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int j0 = 8 * k + KF::PERM[2 * jj], j1 = 8 * k + KF::PERM[2 * jj + 1];
                mul_split(qh[4 * k + jj], qf[j0], qf[j1], sp[jj], bh.u[jj], bl.u[jj]);
                bz = mix_lo(zp[jj], qf[j0], bz);
                bz = mix_hi(zp[jj], qf[j1], bz);
            }
            Frag a0, a1;
            KF::template get<k>(P.kw[0], a0);
            KF::template get<k>(P.kw[1], a1);
            c0 = mfma(a0, bh, c0);
            c0 = mfma(a0, bl, c0);
            c1 = mfma(a1, bh, c1);
            c1 = mfma(a1, bl, c1);
            if constexpr (k + 1 < NCH) spc = spn, zpc = zpn;
            __builtin_amdgcn_sched_barrier(0);
        });
        const float bias = col4_sum(bz * ((float)(1 << KSH) / (float)(1 << 8)));
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = fmaf(c0[i], kTwo16, bias);
            sc[4 + i] = fmaf(c1[i], kTwo16, bias);
        }
    };

    // Partial scores of a residual tile (keys kept in the input dtype): keys and
    // queries both split into fp16 hi + lo parts (three MFMAs).
    auto key_scores_resid = [&](int t0, float* sc) {
        f32x4 c[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        static_for<NCH>([&](auto K) {
            constexpr int k = K;
            const int cb = cw0 + lg * DQ + 8 * k;
            Frag bh, bl;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float x0 = qf[8 * k + 2 * jj] * ((float)(1 << KSH) / (float)(1 << 8));
                const float x1 = qf[8 * k + 2 * jj + 1] * ((float)(1 << KSH) / (float)(1 << 8));
                split2(x0, x1, bh.u[jj], bl.u[jj]);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int t = min(t0 + 8 * (ln >> 2) + 4 * s + (ln & 3), wb - 1);
                float kv[8];
                load8_rt(kr, (size_t)(t & (Gk - 1)) * D + cb, a.in_dtype, kv);
                Frag ah, al;
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) split2(kv[2 * jj], kv[2 * jj + 1], ah.u[jj], al.u[jj]);
                c[s] = mfma(ah, bh, c[s]);
                c[s] = mfma(ah, bl, c[s]);
                c[s] = mfma(al, bh, c[s]);
            }
        });
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            sc[i] = c[0][i];
            sc[4 + i] = c[1][i];
        }
    };

    // Sum the waves' partial scores (fixed order: identical in every wave), mask.
    auto full_scores = [&](float* sc, int buf, int t0, int lim) {
        if constexpr (NWV > 1) {
            float* xs = xbuf + (size_t)buf * NWV * 512;
            *(float4*)&xs[(wave * 64 + lane) * 8] = make_float4(sc[0], sc[1], sc[2], sc[3]);
            *(float4*)&xs[(wave * 64 + lane) * 8 + 4] = make_float4(sc[4], sc[5], sc[6], sc[7]);
            wg_lds_barrier();
#pragma unroll
            for (int j = 0; j < 8; ++j) sc[j] = 0.f;
#pragma unroll
            for (int w = 0; w < NWV; ++w) {
                const float4 u0 = *(const float4*)&xs[(w * 64 + lane) * 8];
                const float4 u1 = *(const float4*)&xs[(w * 64 + lane) * 8 + 4];
                sc[0] += u0.x, sc[1] += u0.y, sc[2] += u0.z, sc[3] += u0.w;
                sc[4] += u1.x, sc[5] += u1.y, sc[6] += u1.z, sc[7] += u1.w;
            }
        }
#pragma unroll
        for (int j = 0; j < 8; ++j)
            if (t0 + 8 * lg + j >= lim) sc[j] = -INFINITY;
    };

    // Softmax weights of the tile and the value products of this wave's channels.
    auto values = [&](const float* sc) {
        float tmax = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
        tmax = col4_max(tmax);
        if (__builtin_amdgcn_ballot_w64(tmax > m)) {
            const float mnew = fmaxf(m, tmax);
            const float alpha = __builtin_amdgcn_exp2f(m - mnew);
            // row 4lg + i of the accumulators belongs to query 4lg + i
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * lg + i);
#pragma unroll
                for (int n = 0; n < NSUB; ++n) acc[n][i] *= ai;
                cz[i] *= ai;
            }
            m = mnew;
        }
        if (kb_tile < kb) {  // a tile with larger value steps: lower the exponent (exact rescale)
            const float f = __builtin_amdgcn_ldexpf(1.0f, kb_tile - kb);
#pragma unroll
            for (int n = 0; n < NSUB; ++n) acc[n] *= f;
            kb = kb_tile;
        }
        // p <= 1 (exact running maximum), kept in fp16 range with power-of-two
        // scales: 2^kb for the value product, 2^KZ for zero points / denominator
        float p[8];
        const float mb = m - (float)kb;
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(sc[j] - mb);
        Frag ph, pl, pb;  // 2^KZ p as hi + lo; 2^KB p truncated to fp16 pairs
        {
            Frag zf;
            float pz[8];
            const float zscale = __builtin_amdgcn_ldexpf(1.0f, KZ - kb);
#pragma unroll
            for (int j = 0; j < 8; ++j) pz[j] = p[j] * zscale;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                split2(pz[2 * jj], pz[2 * jj + 1], ph.u[jj], pl.u[jj]);
                pb.u[jj] = pk_rtz(p[2 * jj], p[2 * jj + 1]);
            }
            const uint4 z4 = *(const uint4*)&zt_lds[wave][ln][8 * lg];
            zf.u[0] = z4.x, zf.u[1] = z4.y, zf.u[2] = z4.z, zf.u[3] = z4.w;
            cz = mfma(ph, zf, cz);
            cz = mfma(pl, zf, cz);
        }
        // Output tiles 2b, 2b+1 take columns 32b + 2ln and 32b + 2ln + 1 of the
        // wave's value tile: one 16-bit LDS read per token row feeds both.
        const uint8_t* vt = &vt_lds[wave][8 * lg * VROW + 2 * ln];
        uint32_t vb[2][8];
        uint4 sv[2];
        auto read_v = [&](int b, uint32_t* w, uint4& s4) {
#pragma unroll
            for (int j = 0; j < 8; ++j) w[j] = *(const uint16_t*)&vt[j * VROW + 32 * b];
            s4 = *(const uint4*)&st_lds[wave][(32 * b) >> lgv][8 * lg];
        };
        read_v(0, vb[0], sv[0]);
        Frag sh, sl;
        static_for<NSUB / 2>([&](auto B) {
            constexpr int b = B;
            if constexpr (b + 1 < NSUB / 2) read_v(b + 1, vb[(b + 1) & 1], sv[(b + 1) & 1]);
            if ((b & ((1 << bpg) - 1)) == 0) {  // first block of a value group: P' = p * s
                const uint32_t sw[4] = {sv[b & 1].x, sv[b & 1].y, sv[b & 1].z, sv[b & 1].w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj) mul_split(pb.u[jj], p[2 * jj], p[2 * jj + 1], sw[jj], sh.u[jj], sl.u[jj]);
            }
            // code << VSH in each half: the high byte for 2- and 3-bit codes,
            // else the low byte shifted
            const uint32_t* w = vb[b & 1];
            Frag f0, f1;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                if constexpr (VSH == 8) {
                    f0.u[jj] = __builtin_amdgcn_perm(w[2 * jj + 1], w[2 * jj], 0x040c000cu);
                    f1.u[jj] = __builtin_amdgcn_perm(w[2 * jj + 1], w[2 * jj], 0x050c010cu);
                } else {
                    f0.u[jj] = __builtin_amdgcn_perm(w[2 * jj + 1], w[2 * jj], 0x0c040c00u) << VSH;
                    f1.u[jj] = __builtin_amdgcn_perm(w[2 * jj + 1], w[2 * jj], 0x0c050c01u) << VSH;
                }
            }
            acc[2 * b] = mfma(sh, f0, acc[2 * b]);
            acc[2 * b] = mfma(sl, f0, acc[2 * b]);
            acc[2 * b + 1] = mfma(sh, f1, acc[2 * b + 1]);
            acc[2 * b + 1] = mfma(sl, f1, acc[2 * b + 1]);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ---- tiles of the split, shared by all waves
    const int ntile = (wb - wa + 31) >> 5;
    const int nqt = qend > wa ? (qend - wa + 31) >> 5 : 0;
#pragma unroll
    for (int b = 0; b < 2; ++b) {
        if (b < nqt) {
            load_kmeta(pf[b], wa + 32 * b);
            load_values(pf[b], wa + 32 * b);
            load_keys(pf[b], wa + 32 * b);
        }
    }
    wave_lds_sync();  // constant zero-point rows written
    // Tile i uses set i & 1 and refills it with tile i + 2 (the last tile is
    // repeated past the end: cache hits).
    auto quant_tile = [&](Pref& P, int i) {
        const int t0 = wa + 32 * i;
        const int tn = wa + 32 * min(i + 2, nqt - 1);
        stage(P, true);
        load_kmeta(P, tn);
        load_values(P, tn);
        __builtin_amdgcn_sched_barrier(0);  // issue the prefetch before any use of the key words
        wave_lds_sync();
        float sc[8];
        key_scores_quant(P, sc);
        load_keys(P, tn);
        full_scores(sc, i & 1, t0, qend);
        values(sc);
        wave_lds_sync();  // the next stage rewrites this wave's LDS tiles
    };
    for (int i = 0; i < nqt; i += 2) {
        quant_tile(pf[0], i);
        if (i + 1 < nqt) quant_tile(pf[1], i + 1);
    }
    for (int i = nqt; i < ntile; ++i) {
        const int t0 = wa + 32 * i;
        load_values(pf[0], t0);
        stage(pf[0], false);
        wave_lds_sync();
        float sc[8];
        key_scores_resid(t0, sc);
        full_scores(sc, i & 1, t0, wb);
        values(sc);
        wave_lds_sync();
    }

    // ---- this split's partial (m, l, o) for the R real queries: o = 2^24 acc + zero-point sums
    float* o_lds = xbuf + wave * 16 * DW;  // [16][DW] by value-tile position
    if constexpr (NWV > 1) wg_lds_barrier();  // every wave is done reading the partial scores
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
#pragma unroll
        for (int b = 0; b < NSUB / 2; ++b) {
            // zero-point sum of (r, group), carrying 2^KZ
            const float zs = __shfl(cz[i], 16 * lg + ((32 * b) >> lgv)) * (1.0f / (float)(1 << KZ));
            const float oscale = __builtin_amdgcn_ldexpf(1.0f, 24 - kb - VSH);
            o_lds[r * DW + 32 * b + 2 * ln] = fmaf(acc[2 * b][i], oscale, zs);
            o_lds[r * DW + 32 * b + 2 * ln + 1] = fmaf(acc[2 * b + 1][i], oscale, zs);
        }
    }
    wave_lds_sync();
    for (int i = lane; i < R * DW; i += 64) {
        const int r = i / DW, pos = i % DW;
        const size_t slot = ((size_t)seq * a.q_heads + kvh * R + r) * a.max_chunks + split;
        a.ws_o[slot * D + cw0 + val_chan<BV>(pos)] = o_lds[r * DW + pos];
    }
    if (wave == 0) {
        // denominator of query 4lg + i sits in column ngw of cz
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int r = 4 * lg + i;
            if (ln == ngw && r < R) {
                const size_t slot = ((size_t)seq * a.q_heads + kvh * R + r) * a.max_chunks + split;
                a.ws_ml[slot * 2 + 1] = cz[i] * (1.0f / (float)(1 << KZ));
            }
        }
        if (lg == 0 && ln < R) {
            const size_t slot = ((size_t)seq * a.q_heads + kvh * R + ln) * a.max_chunks + split;
            a.ws_ml[slot * 2 + 0] = m;
        }
    }
}

template <int D, int BK>
hipError_t gqa_bv(const DecodeArgs& a, int bv, dim3 grid, hipStream_t s) {
    const dim3 block(D / wave_channels<BK>() * 64);
    switch (bv) {
        case 2: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 2>), grid, block, 0, s, a); break;
        case 3: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 3>), grid, block, 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 4>), grid, block, 0, s, a); break;
        case 6: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 6>), grid, block, 0, s, a); break;
        default: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 8>), grid, block, 0, s, a); break;
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

// Compiled once per head_dim (KVQ_GQA_HEAD_DIM = 64, 128, 256).
#define KVQ_GCAT2(a, b) a##b
#define KVQ_GCAT(a, b) KVQ_GCAT2(a, b)
hipError_t KVQ_GCAT(launch_decode_gqa_d, KVQ_GQA_HEAD_DIM)(const DecodeArgs& a, int bits_k, int bits_v, int nseqs,
                                                           hipStream_t s) {
    // x: the quantized splits only (the workspace's full-precision slots have no
    // workgroups here: empty ones would leave the busy ones on a few XCDs)
    dim3 grid(a.max_chunks - a.win_splits, a.kv_heads, nseqs * a.n_layers);
    return gqa_bk<KVQ_GQA_HEAD_DIM>(a, bits_k, bits_v, grid, s);
}

}  // namespace kvq
