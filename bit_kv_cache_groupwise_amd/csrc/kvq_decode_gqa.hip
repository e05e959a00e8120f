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
// Per wave, tiles of 32 tokens (one key block when G = 32):
//   scores^T[t][r] = 2^-16 * sum_c A[t][c] B[c][r] + bias_b[r], with
//     A = key codes of token t (fp16 subnormals code * 2^(sh-24), unpacked
//         from the lane's own row bits, exact),
//     B = (q_r,c * s_b,c) * 2^(8-sh) in fp16 hi + lo parts (two MFMAs),
//     bias_b[r] = sum_c q_r,c z_b,c;
//   out[r][c] = 2^24 * sum_t P'[r][t] V[t][c] + sum_t p_rt z_t,g(c), with
//     P' = p * s_t,g in fp16 hi + lo, V = value codes as fp16 subnormals read
//     transposed from an LDS byte tile.
// The score output layout (lane: 4 tokens x 1 query) is exactly the operand
// layout the value product needs for P (8 tokens x 1 query per lane), so the
// softmax weights never leave registers. Online softmax with an exact running
// maximum (P' must stay inside fp16 range). Splits are merged by merge_kernel.
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

__device__ __forceinline__ uint32_t f16_bits(float x) { return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)x); }

// x ~= hi + lo with both halves fp16 (round to nearest even each).
__device__ __forceinline__ void split_pair(float x0, float x1, uint32_t& hi, uint32_t& lo) {
    const _Float16 h0 = (_Float16)x0, h1 = (_Float16)x1;
    hi = (uint32_t)__builtin_bit_cast(uint16_t, h0) | ((uint32_t)__builtin_bit_cast(uint16_t, h1) << 16);
    lo = f16_bits(x0 - (float)h0) | (f16_bits(x1 - (float)h1) << 16);
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

// 3- and 6-bit codes straddle words: one bit-field extract per code.
template <int B>
struct KeyFragStraddle {
    static constexpr int PERM[8] = {0, 1, 2, 3, 4, 5, 6, 7};
    static constexpr int SHIFT[8] = {0, 0, 0, 0, 0, 0, 0, 0};
    template <int J>
    static __device__ __forceinline__ uint32_t code(const uint32_t* w) {
        constexpr int pos = J * B, wi = pos >> 5, sh = pos & 31;
        if constexpr (sh + B <= 32) return (w[wi] >> sh) & ((1u << B) - 1u);
        else return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << B) - 1u);
    }
    template <int K>
    static __device__ __forceinline__ void get(const uint32_t* w, Frag& f) {
        f.u[0] = code<8 * K + 0>(w) | (code<8 * K + 1>(w) << 16);
        f.u[1] = code<8 * K + 2>(w) | (code<8 * K + 3>(w) << 16);
        f.u[2] = code<8 * K + 4>(w) | (code<8 * K + 5>(w) << 16);
        f.u[3] = code<8 * K + 6>(w) | (code<8 * K + 7>(w) << 16);
    }
};
template <>
struct KeyFrag<3> : KeyFragStraddle<3> {};
template <>
struct KeyFrag<6> : KeyFragStraddle<6> {};

// Code j (0..31) of one packed 32-channel unit.
template <int B, int J>
__device__ __forceinline__ uint32_t unit_code(const uint32_t* w) {
    constexpr int pos = J * B, wi = pos >> 5, sh = pos & 31;
    if constexpr (sh + B <= 32) return (w[wi] >> sh) & ((1u << B) - 1u);
    else return __builtin_amdgcn_alignbit(w[wi + 1], w[wi], sh) & ((1u << B) - 1u);
}

template <int B, int J>
__device__ __forceinline__ void unit_bytes(const uint32_t* w, uint32_t* out) {
    if constexpr (J < 8) {
        out[J] = unit_code<B, 4 * J>(w) | (unit_code<B, 4 * J + 1>(w) << 8) | (unit_code<B, 4 * J + 2>(w) << 16) |
                 (unit_code<B, 4 * J + 3>(w) << 24);
        unit_bytes<B, J + 1>(w, out);
    }
}

template <int CTRL>
__device__ __forceinline__ float dppf(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

// Reductions over the 16 lanes of a row (lanes that share l / 16).
__device__ __forceinline__ float row16_max(float v) {
    v = fmaxf(v, dppf<0xb1>(v));
    v = fmaxf(v, dppf<0x4e>(v));
    v = fmaxf(v, dppf<0x141>(v));
    v = fmaxf(v, dppf<0x140>(v));
    return v;
}
// Reductions over the 4 lanes that share l % 16 (lanes l, l^16, l^32, l^48).
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

__device__ __forceinline__ float load_in_rt2(const void* p, size_t i, int dt) {
    if (dt == 0) return load_in<0>(p, i);
    if (dt == 1) return load_in<1>(p, i);
    return load_in<2>(p, i);
}

constexpr float kTwo16 = 65536.0f;
constexpr float kTwo24 = 16777216.0f;

template <int D, int BK, int BV>
__global__ __launch_bounds__(256) void decode_gqa_kernel(DecodeArgs a) {
    constexpr int NW = 4, NT = 256;
    constexpr int DQ = D / 4;          // channels of one lane group in the key contraction
    constexpr int NCH = D / 32;        // MFMA chunks over channels
    constexpr int NSUB = D / 16;       // value column tiles
    constexpr int KWL = DQ * BK / 32;  // key words per lane per token
    constexpr int VROW = D + 4;        // bytes per row of the value tile (padded)
    using KF = KeyFrag<BK>;

    __shared__ float q_lds[16][D + 4];                        // scaled queries, rows >= R are zero
    __shared__ __align__(16) uint32_t km_lds[NW][D];          // metadata of the current key block
    __shared__ __align__(16) uint8_t vt_lds[NW][32 * VROW];   // value codes of the tile, one byte each
    __shared__ uint32_t vm_lds[NW][32 * 8];                   // value metadata of the tile [token][group]
    __shared__ float z_lds[NW][16][8];                        // per-wave zero-point sums
    __shared__ float ml_lds[NW][16][2];                       // per-wave (m, l)

    const int seq = a.seq_list ? a.seq_list[blockIdx.z] : (int)blockIdx.z;
    const int kvh = blockIdx.y, split = blockIdx.x;
    const int len = a.len[seq];
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    const int R = a.q_heads / a.kv_heads;
    const int CW = a.chunk;
    const int wa = split * CW;
    if (wa >= len) return;  // merge_kernel sees ceil(len / CW) splits
    const int wb = min(wa + CW, len);
    const SeqEntry& e = a.table[seq];
    const int lgk = a.log2_group_k, lgv = a.log2_group_v;
    const int Gk = 1 << lgk;
    const int nqk = (len >> lgk) << lgk;
    const int qend = min(wb, nqk);
    const int vgpr = D >> lgv;  // value groups per row (at most 8)
    const int ln = lane & 15, lg = lane >> 4;

    const uint8_t* kc = a.codes + e.codes[0] + (size_t)kvh * e.codes_hs[0];
    const uint32_t* km = (const uint32_t*)(a.meta + e.meta[0] + (size_t)kvh * e.meta_hs[0]);
    const uint8_t* kr = a.resid + e.resid[0] + (size_t)kvh * e.resid_hs[0];
    const uint8_t* vc = a.codes + e.codes[1] + (size_t)kvh * e.codes_hs[1];
    const uint32_t* vm = (const uint32_t*)(a.meta + e.meta[1] + (size_t)kvh * e.meta_hs[1]);

    for (int i = tid; i < 16 * D; i += NT) {
        const int r = i / D, c = i % D;
        q_lds[r][c] = r < R ? load_in_rt2(a.q, ((size_t)seq * a.q_heads + kvh * R + r) * D + c, a.in_dtype) * a.qscale
                            : 0.f;
    }
    __syncthreads();

    // Lane (ln, lg): softmax state of query ln (replicated over lg); output
    // accumulators O[query 4*lg + i][channel 16*n + ln].
    f32x4 acc[NSUB];
#pragma unroll
    for (int n = 0; n < NSUB; ++n) acc[n] = f32x4{0.f, 0.f, 0.f, 0.f};
    float zacc[8];
#pragma unroll
    for (int g = 0; g < 8; ++g) zacc[g] = 0.f;
    float m = -INFINITY, lsum = 0.f;
    Frag bhi[NCH], blo[NCH];  // key-side operand q_ln * s_b for the current block
    float bias = 0.f;         // q_ln . z_b
    int cur_block = -1;

    auto wave_lds_sync = [] {
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
    };

    for (int t0 = wa + 32 * wave; t0 < wb; t0 += 32 * NW) {
        const bool quantized = t0 < nqk;  // tiles never straddle nqk (a multiple of G >= 32)
        // ---- stage the tile's value codes (one byte each) and value metadata in LDS
        for (int u = lane; u < 32 * (D / 32); u += 64) {
            const int tt = u / (D / 32), uu = u % (D / 32);
            const int t = min(t0 + tt, wb - 1);
            const uint32_t* src = (const uint32_t*)(vc + (size_t)t * (D * BV / 8)) + uu * BV;
            uint32_t w[BV];
#pragma unroll
            for (int k = 0; k < BV; ++k) w[k] = src[k];
            uint32_t bytes[8];
            if constexpr (BV == 8) {
#pragma unroll
                for (int k = 0; k < 8; ++k) bytes[k] = w[k];
            } else {
                unit_bytes<BV, 0>(w, bytes);
            }
            uint32_t* dst = (uint32_t*)&vt_lds[wave][tt * VROW + uu * 32];  // rows are 4-byte aligned
#pragma unroll
            for (int k = 0; k < 8; ++k) dst[k] = bytes[k];
        }
        for (int i = lane; i < 32 * vgpr; i += 64) {
            const int t = min(t0 + i / vgpr, wb - 1);
            vm_lds[wave][i] = vm[(size_t)t * vgpr + i % vgpr];
        }
        // ---- key scores: lane holds query ln of tokens 16*s + 4*lg + i  (sc[4*s + i])
        float sc[8];
        if (quantized) {
            const int b = t0 >> lgk;
            if (b != cur_block) {
                cur_block = b;
                for (int i = lane; i < D; i += 64) km_lds[wave][i] = km[(size_t)b * D + i];
                wave_lds_sync();
                float bz = 0.f;
#pragma unroll
                for (int k = 0; k < NCH; ++k) {
                    const int c0 = lg * DQ + 8 * k;
                    float qv[8];
                    uint32_t mv[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        qv[j] = q_lds[ln][c0 + j];
                        mv[j] = km_lds[wave][c0 + j];
                    }
                    float v[8];
#pragma unroll
                    for (int j = 0; j < 8; ++j) {
                        const int cj = KF::PERM[j];
                        v[j] = qv[cj] * f16_to_f32(mv[cj]) * (float)(1 << (8 - KF::SHIFT[j]));
                        bz = fmaf(qv[j], f16_to_f32(mv[j] >> 16), bz);
                    }
                    split_pair(v[0], v[1], bhi[k].u[0], blo[k].u[0]);
                    split_pair(v[2], v[3], bhi[k].u[1], blo[k].u[1]);
                    split_pair(v[4], v[5], bhi[k].u[2], blo[k].u[2]);
                    split_pair(v[6], v[7], bhi[k].u[3], blo[k].u[3]);
                }
                bias = col4_sum(bz);
            }
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const int t = min(t0 + 16 * s + ln, nqk - 1);
                uint32_t w[KWL];
                const uint32_t* src = (const uint32_t*)(kc + (size_t)t * (D * BK / 8)) + lg * KWL;
#pragma unroll
                for (int k = 0; k < KWL; ++k) w[k] = src[k];
                f32x4 c = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
                for (int k = 0; k < NCH; ++k) {
                    Frag af;
                    if constexpr (NCH > 0) {
                        if (k == 0) KF::template get<0>(w, af);
                        if (k == 1) KF::template get<1 % (NCH > 1 ? NCH : 1)>(w, af);
                        if (k == 2) KF::template get<2 % (NCH > 2 ? NCH : 1)>(w, af);
                        if (k == 3) KF::template get<3 % (NCH > 3 ? NCH : 1)>(w, af);
                        if (k == 4) KF::template get<4 % (NCH > 4 ? NCH : 1)>(w, af);
                        if (k == 5) KF::template get<5 % (NCH > 5 ? NCH : 1)>(w, af);
                        if (k == 6) KF::template get<6 % (NCH > 6 ? NCH : 1)>(w, af);
                        if (k == 7) KF::template get<7 % (NCH > 7 ? NCH : 1)>(w, af);
                    }
                    c = mfma(af, bhi[k], c);
                    c = mfma(af, blo[k], c);
                }
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int tt = t0 + 16 * s + 4 * lg + i;
                    sc[4 * s + i] = tt < qend ? c[i] * kTwo16 + bias : -INFINITY;
                }
            }
        } else {
            // residual key rows in the input dtype (fewer than G tokens): VALU dot products
#pragma unroll
            for (int j = 0; j < 8; ++j) {
                const int tt = t0 + (j < 4 ? 4 * lg + j : 16 + 4 * lg + j - 4);
                float d = -INFINITY;
                if (tt < wb) {
                    const size_t base = (size_t)(tt & (Gk - 1)) * D;
                    d = 0.f;
                    for (int c = 0; c < D; ++c) d = fmaf(q_lds[ln][c], load_in_rt2(kr, base + c, a.in_dtype), d);
                }
                sc[j] = d;
            }
        }
        wave_lds_sync();
        // ---- online softmax for query ln (exact running maximum)
        float tmax = sc[0];
#pragma unroll
        for (int j = 1; j < 8; ++j) tmax = fmaxf(tmax, sc[j]);
        tmax = col4_max(tmax);
        const float mnew = fmaxf(m, tmax);
        const float alpha = m == -INFINITY ? 0.f : exp2f(m - mnew);  // 0 on the first tile, 1 when unchanged
        if (__any(mnew != m)) {
            lsum *= alpha;
#pragma unroll
            for (int g = 0; g < 8; ++g) zacc[g] *= alpha;
            // output row 4*lg + i belongs to query 4*lg + i: fetch that query's factor
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const float ai = __shfl(alpha, 4 * lg + i);
#pragma unroll
                for (int n = 0; n < NSUB; ++n) acc[n][i] *= ai;
            }
            m = mnew;
        }
        float p[8];
#pragma unroll
        for (int j = 0; j < 8; ++j) {
            p[j] = exp2f(sc[j] - m);
            lsum += p[j];
        }
        // ---- values: per value group, P' = p * s (hi, lo) against the codes read transposed from LDS
#pragma unroll
        for (int g = 0; g < 8; ++g) {
            if (g < vgpr) {
                float pv[8];
#pragma unroll
                for (int j = 0; j < 8; ++j) {
                    const int tt = j < 4 ? 4 * lg + j : 16 + 4 * lg + j - 4;
                    const uint32_t w = vm_lds[wave][tt * vgpr + g];
                    pv[j] = p[j] * f16_to_f32(w);
                    zacc[g] = fmaf(p[j], f16_to_f32(w >> 16), zacc[g]);
                }
                Frag ahi, alo;
                split_pair(pv[0], pv[1], ahi.u[0], alo.u[0]);
                split_pair(pv[2], pv[3], ahi.u[1], alo.u[1]);
                split_pair(pv[4], pv[5], ahi.u[2], alo.u[2]);
                split_pair(pv[6], pv[7], ahi.u[3], alo.u[3]);
                const int n0 = (g << lgv) >> 4, n1 = ((g + 1) << lgv) >> 4;  // column tiles of group g
#pragma unroll
                for (int n = 0; n < NSUB; ++n) {
                    if (n >= n0 && n < n1) {
                        const uint8_t* vt = &vt_lds[wave][16 * n + ln];
                        Frag bf;
#pragma unroll
                        for (int h = 0; h < 4; ++h) {
                            const int ta = 2 * h < 4 ? 4 * lg + 2 * h : 16 + 4 * lg + 2 * h - 4;
                            const int tb = ta + 1;
                            bf.u[h] = (uint32_t)vt[ta * VROW] | ((uint32_t)vt[tb * VROW] << 16);
                        }
                        acc[n] = mfma(ahi, bf, acc[n]);
                        acc[n] = mfma(alo, bf, acc[n]);
                    }
                }
            }
        }
        wave_lds_sync();  // the next tile rewrites this wave's LDS tiles
    }

    // ---- per-wave results to LDS: (m, l) and zero-point sums of query ln
    lsum = col4_sum(lsum);
#pragma unroll
    for (int g = 0; g < 8; ++g) zacc[g] = col4_sum(zacc[g]);
    if (lg == 0) {
        ml_lds[wave][ln][0] = m;
        ml_lds[wave][ln][1] = lsum;
#pragma unroll
        for (int g = 0; g < 8; ++g) z_lds[wave][ln][g] = zacc[g];
    }
    __syncthreads();
    // ---- merge the waves into an LDS tile O[16][D] (deterministic order), reusing vt_lds
    float* o_lds = (float*)&vt_lds[0][0];  // 16 * D floats <= sizeof(vt_lds)
    float M[4], wscale[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int r = 4 * lg + i;
        float mm = -INFINITY;
#pragma unroll
        for (int w = 0; w < NW; ++w) mm = fmaxf(mm, ml_lds[w][r][0]);
        M[i] = mm;
        wscale[i] = ml_lds[wave][r][0] == -INFINITY ? 0.f : exp2f(ml_lds[wave][r][0] - mm);
    }
    for (int w = 0; w < NW; ++w) {
        if (wave == w) {
#pragma unroll
            for (int n = 0; n < NSUB; ++n) {
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const int r = 4 * lg + i, c = 16 * n + ln;
                    const float o = (acc[n][i] * kTwo24 + z_lds[wave][r][c >> lgv]) * wscale[i];
                    o_lds[r * D + c] = w == 0 ? o : o_lds[r * D + c] + o;
                }
            }
        }
        __syncthreads();
    }
    // ---- write this split's partial (m, l, o) for the R real queries
    for (int i = tid; i < R * D; i += NT) {
        const int r = i / D, c = i % D;
        const size_t slot = ((size_t)seq * a.q_heads + kvh * R + r) * a.max_chunks + split;
        a.ws_o[slot * D + c] = o_lds[r * D + c];
    }
    if (tid < R) {
        const int r = tid;
        float mm = -INFINITY;
        for (int w = 0; w < NW; ++w) mm = fmaxf(mm, ml_lds[w][r][0]);
        float L = 0.f;
        for (int w = 0; w < NW; ++w)
            if (ml_lds[w][r][0] != -INFINITY) L = fmaf(ml_lds[w][r][1], exp2f(ml_lds[w][r][0] - mm), L);
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
        case 3: return gqa_bv<D, 3>(a, bv, grid, s);
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
    dim3 grid(a.max_chunks, a.kv_heads, nseqs);
    return gqa_bk<KVQ_GQA_HEAD_DIM>(a, bits_k, bits_v, grid, s);
}

}  // namespace kvq
