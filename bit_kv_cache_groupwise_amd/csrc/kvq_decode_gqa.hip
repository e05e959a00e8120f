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
// 4 waves take interleaved 32-token tiles and meet only at the end. Per tile a
// wave computes
//   scores^T[t][r] = 2^16 * sum_c A[t][c] B[c][r] + bias[r],
//     A = key codes of token t as fp16 subnormals code * 2^(sh-24), unpacked
//         from the lane's own row words (exact),
//     B = q'_rc * s_c in fp16 hi + lo parts (two MFMAs), where q' carries the
//         2^(8-sh) that undoes the code shift,
//     bias[r] = sum_c q_rc z_c on the VALU;
//   O[r][c]  += 2^24 * sum_t (p_rt s_t,g(c))[hi + lo] V[t][c],
//     V = value codes as fp16 subnormals, read transposed from an LDS byte tile;
//   Z[r][g]  += sum_t p_rt [hi + lo] * (z_t,g | 1),
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
// Softmax: online in the log2 domain with a lazily moved reference maximum
// (moved when a score exceeds it by more than 2^8, so weights stay <= 256 and
// P * s stays inside the fp16 range). Splits are merged by merge_kernel.
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
// (x0, x1) ~= hi + lo with hi = fp16 truncation and lo = fp16 of the exact rest.
__device__ __forceinline__ void split2(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    hi = pk_rtz(x0, x1);
    lo = pk_rtz(rem_lo(hi, x0), rem_hi(hi, x1));
}

// Key-code fragments: chunk k of a lane's channel range (8 channels) as 8 fp16
// halves. Half j of the fragment holds channel 8k + PERM[j] of the range as the
// integer code << SHIFT[j], i.e. the fp16 subnormal code * 2^(SHIFT[j]-24).
template <int B>
struct KeyFrag;

template <>
struct KeyFrag<2> {
    static constexpr int PERM[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    static constexpr int SHIFT[8] = {0, 0, 2, 2, 4, 4, 6, 6};
    template <int K>
    static __device__ __forceinline__ void get(const uint32_t* w, Frag& f) {
        const uint32_t x = w[K / 2];
        const uint32_t y = (K & 1) ? __builtin_amdgcn_perm(x, x, 0x0c030c02u) : __builtin_amdgcn_perm(x, x, 0x0c010c00u);
        f.u[0] = y & 0x00030003u;
        f.u[1] = y & 0x000c000cu;
        f.u[2] = y & 0x00300030u;
        f.u[3] = y & 0x00c000c0u;
    }
};

template <>
struct KeyFrag<4> {
    static constexpr int PERM[8] = {0, 4, 1, 5, 2, 6, 3, 7};
    static constexpr int SHIFT[8] = {0, 0, 4, 4, 0, 0, 4, 4};
    template <int K>
    static __device__ __forceinline__ void get(const uint32_t* w, Frag& f) {
        const uint32_t x = w[K];
        const uint32_t y = x >> 8;
        f.u[0] = x & 0x000f000fu;
        f.u[1] = x & 0x00f000f0u;
        f.u[2] = y & 0x000f000fu;
        f.u[3] = y & 0x00f000f0u;
    }
};

template <>
struct KeyFrag<8> {
    static constexpr int PERM[8] = {0, 2, 1, 3, 4, 6, 5, 7};
    static constexpr int SHIFT[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    template <int K>
    static __device__ __forceinline__ void get(const uint32_t* w, Frag& f) {
        const uint32_t x0 = w[2 * K], x1 = w[2 * K + 1];
        f.u[0] = x0 & 0x00ff00ffu;
        f.u[1] = __builtin_amdgcn_perm(x0, x0, 0x0c070c05u);
        f.u[2] = x1 & 0x00ff00ffu;
        f.u[3] = __builtin_amdgcn_perm(x1, x1, 0x0c070c05u);
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
    static constexpr int SHIFT[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    template <int K>
    static __device__ __forceinline__ void get(const uint32_t* w, Frag& f) {
        // chunk K covers codes 8K..8K+7 of the lane's range; a 32-code unit is B words
        const uint32_t* u = w + (K / 4) * B;
        constexpr int j0 = 8 * (K % 4);
        f.u[0] = unit_code<B, j0 + 0>(u) | (unit_code<B, j0 + 1>(u) << 16);
        f.u[1] = unit_code<B, j0 + 2>(u) | (unit_code<B, j0 + 3>(u) << 16);
        f.u[2] = unit_code<B, j0 + 4>(u) | (unit_code<B, j0 + 5>(u) << 16);
        f.u[3] = unit_code<B, j0 + 6>(u) | (unit_code<B, j0 + 7>(u) << 16);
    }
};
template <>
struct KeyFrag<3> : KeyFragStraddle<3> {};
template <>
struct KeyFrag<6> : KeyFragStraddle<6> {};

// Shift at which channel offset j (0..7 within an 8-channel window) sits in its
// key fragment half: SHIFT[PERM^-1[j]].
template <int B>
__host__ __device__ constexpr int chan_shift(int j) {
    return B == 2 ? 2 * (j & 3) : B == 4 ? 4 * (j & 1) : 0;
}

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

// Sums and maxima over the 4 lanes that share l % 16 (lanes l, l^16, l^32, l^48).
__device__ __forceinline__ float col4_sum(float v) {
    v += __shfl_xor(v, 16);
    v += __shfl_xor(v, 32);
    return v;
}
__device__ __forceinline__ float col4_max(float v) {
    v = fmaxf(v, __shfl_xor(v, 16));
    v = fmaxf(v, __shfl_xor(v, 32));
    return v;
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

template <int D, int BK, int BV>
__global__ __launch_bounds__(256) void decode_gqa_kernel(DecodeArgs a) {
    constexpr int NW = 4, NT = 256;
    constexpr int DQ = D / 4;            // key channels of one lane group (lg)
    constexpr int NCH = D / 32;          // 8-channel MFMA chunks per lane group
    constexpr int NSUB = D / 16;         // 16-column output tiles
    constexpr int KWL = DQ * BK / 32;    // key words of a lane per token
    constexpr int VROW = D + 8;          // bytes per token row of the value tile
    constexpr int UPL = D / 64;          // value units per lane per tile (32 tokens x D/32 units)
    constexpr int UPR = D / 32;          // value units per token
    constexpr int KM = D / 64;           // key metadata words per lane per block
    constexpr int KALIGN = pow2_align(D * BK / 8) < pow2_align(KWL * 4) ? pow2_align(D * BK / 8) : pow2_align(KWL * 4);
    constexpr int VALIGN = pow2_align(D * BV / 8) < pow2_align(BV * 4) ? pow2_align(D * BV / 8) : pow2_align(BV * 4);
    constexpr int NSH = BK == 2 ? 4 : BK == 4 ? 2 : 1;  // distinct code shifts of the key fragments
    using KF = KeyFrag<BK>;
    static_assert(KWL * 32 == DQ * BK, "lane key range must be whole words");

    __shared__ __align__(16) float q_lds[16][D + 4];         // q * scale * 2^(8 - shift); rows >= R zero
    __shared__ __align__(16) uint32_t km_lds[NW][D];        // key metadata of the tile's block
    __shared__ __align__(16) uint8_t vt_lds[NW][32 * VROW]; // value codes of the tile, one byte each
    __shared__ __align__(16) uint16_t st_lds[NW][8][32];    // value scales [group][token]
    __shared__ __align__(16) uint16_t zt_lds[NW][16][32];   // value zero points [group][token]; row G = 1.0
    __shared__ float xm_lds[NW][16];                        // per-wave reference maxima
    __shared__ float xz_lds[NW][16][16];                    // per-wave zero-point sums and denominators

    const int seq = a.seq_list ? a.seq_list[blockIdx.z] : (int)blockIdx.z;
    const int kvh = blockIdx.y, split = blockIdx.x;
    const int len = a.len[seq];
    const int CW = a.chunk;
    const int wa = split * CW;
    if (wa >= len) return;  // merge_kernel sees ceil(len / CW) splits
    const int wb = min(wa + CW, len);
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int ln = lane & 15, lg = lane >> 4;
    const int R = a.q_heads / a.kv_heads;
    const SeqEntry& e = a.table[seq];
    const int lgk = a.log2_group_k, lgv = a.log2_group_v;
    const int Gk = 1 << lgk;
    const int nqk = (len >> lgk) << lgk;  // tokens with quantized keys
    const int qend = min(wb, nqk);
    const int vgpr = D >> lgv;            // value groups per token (1..8)
    const int tpg = lgv - 4;              // log2 of output tiles per value group

    const uint8_t* kc = a.codes + e.codes[0] + (size_t)kvh * e.codes_hs[0];
    const uint32_t* km = (const uint32_t*)(a.meta + e.meta[0] + (size_t)kvh * e.meta_hs[0]);
    const uint8_t* kr = a.resid + e.resid[0] + (size_t)kvh * e.resid_hs[0];
    const uint8_t* vc = a.codes + e.codes[1] + (size_t)kvh * e.codes_hs[1];
    const uint32_t* vm = (const uint32_t*)(a.meta + e.meta[1] + (size_t)kvh * e.meta_hs[1]);

    // ---- queries: q * scale * 2^(8 - chan_shift(c mod 8)), zero rows for r >= R
    for (int i = tid; i < 16 * (D / 8); i += NT) {
        const int r = i / (D / 8), c = (i % (D / 8)) * 8;
        float v[8];
        if (r < R) {
            load8_rt(a.q, ((size_t)seq * a.q_heads + kvh * R + r) * D + c, a.in_dtype, v);
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j) v[j] = 0.f;
        }
#pragma unroll
        for (int j = 0; j < 8; ++j) q_lds[r][c + j] = v[j] * a.qscale * (float)(1 << (8 - chan_shift<BK>(j)));
    }
    // constant rows of the zero-point fragment: 1.0 in row vgpr, 0 above it
    for (int i = lane; i < 16 * 32; i += 64) {
        const int g = i >> 5;
        if (g >= vgpr) zt_lds[wave][g][i & 31] = g == vgpr ? (uint16_t)0x3c00u : (uint16_t)0u;
    }
    __syncthreads();

    f32x4 acc[NSUB];
#pragma unroll
    for (int n = 0; n < NSUB; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    f32x4 cz = {0.f, 0.f, 0.f, 0.f};  // C[query 4lg+i][col ln]: zero-point sums (ln < vgpr), denominator (ln == vgpr)
    float m = kFarBelow;              // reference maximum of query ln

    // ---- prefetch registers (the tile after the one being computed)
    uint32_t kw[2][KWL];  // key words of token rows 8(ln>>2) + 4s + (ln&3), lane group lg
    uint32_t kmw[KM];     // key metadata words lane*KM.. of the tile's block
    uint32_t vw[UPL][BV]; // value units lane + 64u of the tile
    uint32_t vmw[4];      // value metadata words lane + 64u of the tile

    auto load_keys = [&](int t0) {
#pragma unroll
        for (int s = 0; s < 2; ++s) {
            const int t = min(t0 + 8 * (ln >> 2) + 4 * s + (ln & 3), nqk - 1);
            load_n<KWL, KALIGN>((const uint32_t*)(kc + (size_t)t * (D * BK / 8)) + lg * KWL, kw[s]);
        }
    };
    auto load_kmeta = [&](int t0) {
        load_n<KM, pow2_align(KM * 4)>(km + (size_t)(t0 >> lgk) * D + lane * KM, kmw);
    };
    auto load_values = [&](int t0) {
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int f = lane + 64 * u;
            const int t = min(t0 + f / UPR, wb - 1);
            load_n<BV, VALIGN>((const uint32_t*)(vc + (size_t)t * (D * BV / 8)) + (f % UPR) * BV, vw[u]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int f = lane + 64 * u;
            if (f < 32 * vgpr) {
                const int t = min(t0 + f / vgpr, wb - 1);
                vmw[u] = vm[(size_t)t * vgpr + f % vgpr];
            }
        }
    };
    // Stage value bytes, value scales / zero points and key metadata of the tile in LDS.
    auto stage = [&](bool with_keys) {
#pragma unroll
        for (int u = 0; u < UPL; ++u) {
            const int f = lane + 64 * u;
            uint32_t by[8];
            unit_to_bytes<BV>(vw[u], by);
            uint32_t* dst = (uint32_t*)&vt_lds[wave][(f / UPR) * VROW + (f % UPR) * 32];
#pragma unroll
            for (int k = 0; k < 4; ++k) ((uint2*)dst)[k] = make_uint2(by[2 * k], by[2 * k + 1]);
        }
#pragma unroll
        for (int u = 0; u < 4; ++u) {
            const int f = lane + 64 * u;
            if (f < 32 * vgpr) {
                const int tt = f / vgpr, g = f % vgpr;
                st_lds[wave][g][tt] = (uint16_t)(vmw[u] & 0xffffu);
                zt_lds[wave][g][tt] = (uint16_t)(vmw[u] >> 16);
            }
        }
        if (with_keys) store_lds_n<KM>(&km_lds[wave][lane * KM], kmw);
    };

    // Keys of a quantized tile -> scores sc[j] of query ln, token t0 + 8lg + j.
    auto key_scores_quant = [&](int t0, float* sc) {
        f32x4 c0 = {0.f, 0.f, 0.f, 0.f}, c1 = {0.f, 0.f, 0.f, 0.f};
        float bz[NSH];
#pragma unroll
        for (int h = 0; h < NSH; ++h) bz[h] = 0.f;
        static_for<NCH>([&](auto K) {
            constexpr int k = K;
            const int cb = lg * DQ + 8 * k;
            const float4 qa = *(const float4*)&q_lds[ln][cb];
            const float4 qb = *(const float4*)&q_lds[ln][cb + 4];
            const uint4 ma = *(const uint4*)&km_lds[wave][cb];
            const uint4 mb = *(const uint4*)&km_lds[wave][cb + 4];
            const float q[8] = {qa.x, qa.y, qa.z, qa.w, qb.x, qb.y, qb.z, qb.w};
            const uint32_t mw[8] = {ma.x, ma.y, ma.z, ma.w, mb.x, mb.y, mb.z, mb.w};
            Frag bh, bl;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const int c0i = KF::PERM[2 * jj], c1i = KF::PERM[2 * jj + 1];
                const float x0 = mix_lo(mw[c0i], q[c0i], 0.f);
                const float x1 = mix_lo(mw[c1i], q[c1i], 0.f);
                split2(x0, x1, bh.u[jj], bl.u[jj]);
            }
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int h = NSH == 4 ? (j & 3) : NSH == 2 ? (j & 1) : 0;
                bz[h] = mix_hi(mw[j], q[j], bz[h]);
            }
            Frag a0, a1;
            KF::template get<k>(kw[0], a0);
            KF::template get<k>(kw[1], a1);
            c0 = mfma(a0, bh, c0);
            c0 = mfma(a0, bl, c0);
            c1 = mfma(a1, bh, c1);
            c1 = mfma(a1, bl, c1);
            __builtin_amdgcn_sched_barrier(0);  // bound the live LDS operands to one chunk
        });
        float bias = 0.f;
#pragma unroll
        for (int h = 0; h < NSH; ++h) bias = fmaf(bz[h], 1.0f / (float)(1 << (8 - chan_shift<BK>(h))), bias);
        bias = col4_sum(bias);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int t = t0 + 8 * lg + i;
            sc[i] = t < qend ? fmaf(c0[i], kTwo16, bias) : -INFINITY;
            sc[4 + i] = t + 4 < qend ? fmaf(c1[i], kTwo16, bias) : -INFINITY;
        }
    };

    // Keys of a residual tile (rows kept in the input dtype) -> scores, with
    // keys and queries both split into fp16 hi + lo parts (three MFMAs).
    auto key_scores_resid = [&](int t0, float* sc) {
        f32x4 c[2] = {{0.f, 0.f, 0.f, 0.f}, {0.f, 0.f, 0.f, 0.f}};
        static_for<NCH>([&](auto K) {
            constexpr int k = K;
            const int cb = lg * DQ + 8 * k;
            Frag bh, bl;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float x0 = q_lds[ln][cb + 2 * jj] * (1.0f / (float)(1 << (8 - chan_shift<BK>(2 * jj))));
                const float x1 = q_lds[ln][cb + 2 * jj + 1] * (1.0f / (float)(1 << (8 - chan_shift<BK>(2 * jj + 1))));
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
            const int t = t0 + 8 * lg + i;
            sc[i] = t < wb ? c[0][i] : -INFINITY;
            sc[4 + i] = t + 4 < wb ? c[1][i] : -INFINITY;
        }
    };

    // Softmax weights of the tile and the value products.
    auto values = [&](const float* sc) {
        float tmax = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
        tmax = col4_max(tmax);
        if (__builtin_amdgcn_ballot_w64(tmax > m + 8.0f)) {
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
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) p[j] = __builtin_amdgcn_exp2f(sc[j] - m);
        // zero points and denominator
        {
            Frag ph, pl, zf;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) split2(p[2 * jj], p[2 * jj + 1], ph.u[jj], pl.u[jj]);
            const uint4 z4 = *(const uint4*)&zt_lds[wave][ln][8 * lg];
            zf.u[0] = z4.x, zf.u[1] = z4.y, zf.u[2] = z4.z, zf.u[3] = z4.w;
            cz = mfma(ph, zf, cz);
            cz = mfma(pl, zf, cz);
        }
        Frag sh, sl;
        const uint8_t* vt = &vt_lds[wave][8 * lg * VROW + ln];
        static_for<NSUB>([&](auto N) {
            constexpr int n = N;
            if ((n & ((1 << tpg) - 1)) == 0) {
                const uint4 s4 = *(const uint4*)&st_lds[wave][n >> tpg][8 * lg];
                const uint32_t sw[4] = {s4.x, s4.y, s4.z, s4.w};
#pragma unroll
                for (int jj = 0; jj < 4; ++jj)
                    split2(mix_lo(sw[jj], p[2 * jj], 0.f), mix_hi(sw[jj], p[2 * jj + 1], 0.f), sh.u[jj], sl.u[jj]);
            }
            Frag bf;
#pragma unroll
            for (int jj = 0; jj < 4; ++jj)
                bf.u[jj] = (uint32_t)vt[(2 * jj) * VROW + 16 * n] | ((uint32_t)vt[(2 * jj + 1) * VROW + 16 * n] << 16);
            acc[n] = mfma(sh, bf, acc[n]);
            acc[n] = mfma(sl, bf, acc[n]);
            __builtin_amdgcn_sched_barrier(0);
        });
    };

    // ---- tiles of this wave: t0 = first + 128 i
    const int first = wa + 32 * wave;
    const int nq = first < qend ? (qend - first + 127) >> 7 : 0;
    if (nq > 0) {
        load_kmeta(first);
        load_values(first);
        load_keys(first);
    }
    for (int i = 0; i < nq; ++i) {
        const int t0 = first + 128 * i;
        const int tn = i + 1 < nq ? t0 + 128 : t0;  // the last prefetch repeats the tile (cache hits)
        stage(true);
        load_kmeta(tn);
        load_values(tn);
        wave_lds_sync();
        float sc[8];
        key_scores_quant(t0, sc);
        load_keys(tn);
        values(sc);
        wave_lds_sync();  // the next stage rewrites this wave's LDS tiles
    }
    for (int t0 = first + 128 * nq; t0 < wb; t0 += 128) {
        load_values(t0);
        stage(false);
        wave_lds_sync();
        float sc[8];
        key_scores_resid(t0, sc);
        values(sc);
        wave_lds_sync();
    }

    // ---- per-wave (m, zero-point sums, denominators) to LDS
    if (lg == 0) xm_lds[wave][ln] = m;
#pragma unroll
    for (int i = 0; i < 4; ++i) xz_lds[wave][4 * lg + i][ln] = cz[i];
    __syncthreads();
    // ---- merge the waves into an LDS tile O[16][D] (fixed order), reusing vt_lds
    float* o_lds = (float*)&vt_lds[0][0];  // 16 * D floats <= sizeof(vt_lds)
    float wsc[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
        float mm = kFarBelow;
#pragma unroll
        for (int w = 0; w < NW; ++w) mm = fmaxf(mm, xm_lds[w][r]);
        wsc[i] = __builtin_amdgcn_exp2f(xm_lds[wave][r] - mm);
    }
    for (int w = 0; w < NW; ++w) {
        if (wave == w) {
#pragma unroll
            for (int n = 0; n < NSUB; ++n) {
                const int c = val_chan<BV>(16 * n + ln);
                const int g = (16 * n) >> lgv;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * lg + i;
                    const float o = fmaf(acc[n][i], kTwo24, xz_lds[wave][r][g]) * wsc[i];
                    o_lds[r * D + c] = w == 0 ? o : o_lds[r * D + c] + o;
                }
            }
        }
        __syncthreads();
    }
    // ---- this split's partial (m, l, o) for the R real queries
    for (int i = tid; i < R * D; i += NT) {
        const int r = i / D, c = i % D;
        const size_t slot = ((size_t)seq * a.q_heads + kvh * R + r) * a.max_chunks + split;
        a.ws_o[slot * D + c] = o_lds[r * D + c];
    }
    if (tid < R) {
        const int r = tid;
        float mm = kFarBelow;
        for (int w = 0; w < NW; ++w) mm = fmaxf(mm, xm_lds[w][r]);
        float L = 0.f;
        for (int w = 0; w < NW; ++w) L = fmaf(xz_lds[w][r][vgpr], __builtin_amdgcn_exp2f(xm_lds[w][r] - mm), L);
        const size_t slot = ((size_t)seq * a.q_heads + kvh * R + r) * a.max_chunks + split;
        a.ws_ml[slot * 2 + 0] = mm;
        a.ws_ml[slot * 2 + 1] = L;
    }
}

template <int D, int BK>
hipError_t gqa_bv(const DecodeArgs& a, int bv, dim3 grid, hipStream_t s) {
    switch (bv) {
        case 2: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 2>), grid, dim3(256), 0, s, a); break;
        case 3: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 3>), grid, dim3(256), 0, s, a); break;
        case 4: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 4>), grid, dim3(256), 0, s, a); break;
        case 6: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 6>), grid, dim3(256), 0, s, a); break;
        default: hipLaunchKernelGGL((decode_gqa_kernel<D, BK, 8>), grid, dim3(256), 0, s, a); break;
    }
    return hipGetLastError();
}

template <int D>
hipError_t gqa_bk(const DecodeArgs& a, int bk, int bv, dim3 grid, hipStream_t s) {
    switch (bk) {
        case 2: return gqa_bv<D, 2>(a, bv, grid, s);
        case 3:
            if constexpr ((D / 4) * 3 % 32 == 0) return gqa_bv<D, 3>(a, bv, grid, s);
            else return hipErrorInvalidValue;
        case 4: return gqa_bv<D, 4>(a, bv, grid, s);
        case 6:
            if constexpr ((D / 4) * 6 % 32 == 0) return gqa_bv<D, 6>(a, bv, grid, s);
            else return hipErrorInvalidValue;
        default: return gqa_bv<D, 8>(a, bv, grid, s);
    }
}

}  // namespace

// Compiled once per head_dim (KVQ_GQA_HEAD_DIM = 64, 128, 256).
#define KVQ_GCAT2(a, b) a##b
#define KVQ_GCAT(a, b) KVQ_GCAT2(a, b)
hipError_t KVQ_GCAT(launch_decode_gqa_d, KVQ_GQA_HEAD_DIM)(const DecodeArgs& a, int bits_k, int bits_v, int nseqs,
                                                           hipStream_t s) {
    dim3 grid(a.max_chunks, a.kv_heads, nseqs);
    return gqa_bk<KVQ_GQA_HEAD_DIM>(a, bits_k, bits_v, grid, s);
}

}  // namespace kvq
