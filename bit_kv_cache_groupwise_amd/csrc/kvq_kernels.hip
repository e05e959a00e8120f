// HIP kernels of libkvq for CDNA4 (gfx950): groupwise asymmetric quantization
// of KV-cache rows into bit-packed uint32 words, the fused split-K decode
// attention that reads them, the split merge, and the unfused dequantizer.
//
// Sources, by page title and section:
//   [N] nalar.dev, "Kuantisasi KV cache untuk mengurangi memory inferensi long-context"
//   [U] unite.ai (pt), "O Seu Cache KV Nao Tem um Problema de Bits. Tem um Problema de Geometria."
//
// Numerics of the quantizer (must match the published definition bit for
// bit, so this file is compiled with -ffp-contract=off, correctly rounded
// fp32 division and fp32 denormals kept):
//   zero = group min; step = (max - min) / (2^B - 1) as an fp32 subtract then
//   an fp32 divide ([U] "O Que o Erro de Quantizacao E Realmente Feito");
//   both rounded to fp16 (v_cvt_f16_f32, nearest-even); code =
//   clamp(rint((x - z) / s), 0, 2^B - 1) against the stored z, s
//   (v_rndne_f32: ties to even); stored step 0 -> code 0.
#include <hip/hip_runtime.h>

#include <algorithm>

#include "kvq_append.h"
#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace {

using namespace dev;

// ---------------------------------------------------------------------------
// Quantize, channel axis: one group = one channel over a block of G tokens
// ([U] "Chaves: Outliers Tem Endereco Fixo"; [N] "Kuantisasi dapat memindahkan
// pekerjaan ke decode path": rows wait in the residual until the block is
// complete). Workgroup `item` < nb quantizes block b_first + item: the
// workgroup's 256 threads are (token part, channel pair) with the parts a power
// of two; loads are issued 2 tokens at a time, min/max meet in LDS, codes go through
// an LDS [G][D] byte tile and are packed per 32-channel unit. Workgroup 0 also
// copies the rows past the last complete block into the residual (after its
// own reads of the old residual rows).
// LDS: max(G*D bytes of codes, 4*kThreads floats of min/max exchange).
// ---------------------------------------------------------------------------
// Two consecutive channels c, c+1 of token t (even c), from the residual rows
// (t < len0) or the new rows; f32 input takes one channel (the second is unused).
template <int DT>
__device__ __forceinline__ void chan_pair(const TensorArgs& a, const uint8_t* resid, int t, int len0, int row_start,
                                          int head, int c, float& x0, float& x1) {
    const int D = a.head_dim;
    const size_t i = t < len0 ? (size_t)(t % a.group) * D + c
                              : ((size_t)(row_start + t - len0) * a.kv_heads + head) * D + c;
    const void* base = t < len0 ? (const void*)resid : a.src;
    if constexpr (DT == 0) {
        x0 = ((const float*)base)[i];
        x1 = x0;
    } else {
        const uint32_t w = *(const uint32_t*)((const uint16_t*)base + i);
        x0 = half_to_f32<DT>(w & 0xffffu);
        x1 = half_to_f32<DT>(w >> 16);
    }
}

template <int DT>
__device__ __forceinline__ void channel_axis_part(const TensorArgs& a, int item, int head, int seq, uint32_t* smem) {
    const int D = a.head_dim, UPR = D >> 5, G = a.group;
    const int len0 = a.len_in[seq];
    const int n = a.n_new ? a.n_new[seq] : a.n_uniform;
    const int len1 = len0 + n;
    if (a.len_out && item == 0 && head == 0 && threadIdx.x == 0) a.len_out[seq] = len1;
    const int b_first = len0 / G, b_end = len1 / G, nb = b_end - b_first;
    if (item >= (nb > 0 ? nb : 1)) return;
    const int row_start = a.row_start ? a.row_start[seq] : seq * a.n_uniform;
    const SeqEntry& e = a.table[seq];
    const int T = a.tensor, B = e.bits[T];
    const uint8_t* resid = a.resid + e.resid[T] + (size_t)head * e.resid_hs[T];
    constexpr int IB = In<DT>::bytes;

    if (item < nb) {
        // Thread = (token part, channel pair): a token row is D / CPT threads,
        // with 2-byte inputs a 4-byte load per thread; parts = a power of two.
        constexpr int CPT = IB == 4 ? 1 : 2;
        uint8_t* lds_codes = (uint8_t*)smem;
        const int rt = D / CPT;
        const int parts = 1 << (31 - __builtin_clz(kThreads / rt));
        const int part = threadIdx.x / rt, c = (threadIdx.x % rt) * CPT;
        const bool active = part < parts;  // head_dim not dividing 256 leaves threads idle
        const int tpp = G / parts;         // tokens per part, even
        float* lmn = (float*)smem;         // [parts][D] min/max exchange, then reused by the code tile
        float* lmx = lmn + parts * D;
        const int b = b_first + item;
        const float L = (float)((1 << B) - 1);
        const int t0 = b * G + part * tpp;
        float mn0 = INFINITY, mx0 = -INFINITY, mn1 = INFINITY, mx1 = -INFINITY;
        for (int i = 0; active && i < tpp; i += 2) {
            float x[4];
            chan_pair<DT>(a, resid, t0 + i, len0, row_start, head, c, x[0], x[1]);
            chan_pair<DT>(a, resid, t0 + i + 1, len0, row_start, head, c, x[2], x[3]);
            mn0 = fminf(mn0, fminf(x[0], x[2]));
            mx0 = fmaxf(mx0, fmaxf(x[0], x[2]));
            mn1 = fminf(mn1, fminf(x[1], x[3]));
            mx1 = fmaxf(mx1, fmaxf(x[1], x[3]));
        }
        if (active) {
            lmn[part * D + c] = mn0, lmx[part * D + c] = mx0;
            if (CPT == 2) lmn[part * D + c + 1] = mn1, lmx[part * D + c + 1] = mx1;
        }
        __syncthreads();
        for (int p = 0; p < parts; ++p) {
            mn0 = fminf(mn0, lmn[p * D + c]), mx0 = fmaxf(mx0, lmx[p * D + c]);
            if (CPT == 2) mn1 = fminf(mn1, lmn[p * D + c + 1]), mx1 = fmaxf(mx1, lmx[p * D + c + 1]);
        }
        __syncthreads();  // the code tile overwrites the exchange
        const uint32_t sb0 = f32_to_f16_bits((mx0 - mn0) / L), zb0 = f32_to_f16_bits(mn0);
        const uint32_t sb1 = f32_to_f16_bits((mx1 - mn1) / L), zb1 = f32_to_f16_bits(mn1);
        const float s0 = f16_to_f32(sb0), z0 = f16_to_f32(zb0), s1 = f16_to_f32(sb1), z1 = f16_to_f32(zb1);
        const float r0 = quant_rcp(s0), r1 = quant_rcp(s1);
        // the block's page (a block never straddles pages) and its first row there
        const PageRow pr = page_row(a.pages, e, b * G);
        if (active && part == 0) {
            uint32_t* meta = (uint32_t*)(a.meta + pr.base + e.meta[T] + (size_t)head * e.meta_hs[T]);
            meta[(size_t)(pr.row / G) * D + c] = sb0 | (zb0 << 16);
            if (CPT == 2) meta[(size_t)(pr.row / G) * D + c + 1] = sb1 | (zb1 << 16);
        }
        for (int i = 0; active && i < tpp; i += 2) {
            float x[4];
            chan_pair<DT>(a, resid, t0 + i, len0, row_start, head, c, x[0], x[1]);
            chan_pair<DT>(a, resid, t0 + i + 1, len0, row_start, head, c, x[2], x[3]);
            const int r = part * tpp + i;
            if constexpr (CPT == 2) {
                *(uint16_t*)&lds_codes[r * D + c] = (uint16_t)(quant_code(x[0], r0, s0, z0, L) | (quant_code(x[1], r1, s1, z1, L) << 8));
                *(uint16_t*)&lds_codes[(r + 1) * D + c] = (uint16_t)(quant_code(x[2], r0, s0, z0, L) | (quant_code(x[3], r1, s1, z1, L) << 8));
            } else {
                lds_codes[r * D + c] = (uint8_t)quant_code(x[0], r0, s0, z0, L);
                lds_codes[(r + 1) * D + c] = (uint8_t)quant_code(x[2], r0, s0, z0, L);
            }
        }
        __syncthreads();
        uint8_t* codes = a.codes + pr.base + e.codes[T] + (size_t)head * e.codes_hs[T];
        for (int idx = threadIdx.x; idx < G * UPR; idx += kThreads) {
            const int i = idx / UPR, u = idx % UPR;
            const uint32_t* src = smem + (i * D + 32 * u) / 4;
            uint32_t cc[32];
#pragma unroll
            for (int k = 0; k < 8; ++k) {
                const uint32_t v = src[k];
                cc[4 * k + 0] = v & 0xffu;
                cc[4 * k + 1] = (v >> 8) & 0xffu;
                cc[4 * k + 2] = (v >> 16) & 0xffu;
                cc[4 * k + 3] = v >> 24;
            }
            uint32_t* dst = (uint32_t*)(codes + (size_t)(pr.row + i) * (D * B / 8)) + u * B;
            store_codes_rt(B, cc, dst);
        }
    }
    if (item == 0) {
        __syncthreads();  // this block's reads of the old residual rows are done
        residual_rows<DT>(a, head, seq, b_end * G > len0 ? b_end * G : len0, len0, len1, kThreads);
    }
}

// Quantize, channel axis, one wave per block of G tokens, four blocks per
// workgroup: lane l holds channel pairs (2p, 2p + 1), p = l % (64 / HS) +
// (64 / HS) q, of G / HS tokens of the block in registers (HS = 2: lanes l and
// l + 32 hold the two halves of the block, their min and max combined by one
// swap), one coalesced read of each token row, no second pass; min, max, step, zero and codes per channel in
// registers; the codes go through a wave-private LDS tile [G][D] bytes to be
// packed per 32-channel unit. The wave of the append's first block also copies
// the rows past the last complete block into the residual, after its own reads
// of the old residual rows. Same arithmetic and results as channel_axis_part.
template <int DT, int G, int PPL, int HS>
__device__ __forceinline__ void channel_axis_wave(const TensorArgs& a, int item, int head, int seq, uint8_t* smem) {
    constexpr int IB = In<DT>::bytes, NW = IB == 4 ? 2 : 1;  // 32-bit words per channel pair
    constexpr int GL = G / HS, PW = 64 / HS;                 // tokens per lane, pair slots per half
    const int D = a.head_dim, UPR = D >> 5;
    const int len0 = a.len_in[seq];
    const int n = a.n_new ? a.n_new[seq] : a.n_uniform;
    const int len1 = len0 + n;
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    const int lp = lane % PW, t0 = (lane / PW) * GL;  // pair slot, first token of the lane's half
    if (a.len_out && item == 0 && head == 0 && threadIdx.x == 0) a.len_out[seq] = len1;
    const int b_first = len0 / G, b_end = len1 / G, nb = b_end - b_first;
    const int k = item * kQuantBlocksPerGroup + wave;  // block of this append
    if (k >= (nb > 0 ? nb : 1)) return;
    const int row_start = a.row_start ? a.row_start[seq] : seq * a.n_uniform;
    const SeqEntry& e = a.table[seq];
    const int T = a.tensor, B = e.bits[T];
    const uint8_t* resid = a.resid + e.resid[T] + (size_t)head * e.resid_hs[T];
    if (k < nb) {
        const int b = b_first + k;
        const float L = (float)((1 << B) - 1);
        uint32_t raw[GL][PPL][NW];
        // all loads first (pairs past D read channel 0 and are not used)
#pragma unroll
        for (int i = 0; i < GL; ++i) {
            const int t = b * G + t0 + i;
            const uint8_t* row = t < len0 ? resid + (size_t)(t % G) * D * IB
                                          : (const uint8_t*)a.src + ((size_t)(row_start + t - len0) * a.kv_heads + head) * D * IB;
#pragma unroll
            for (int q = 0; q < PPL; ++q) {
                const int c = 2 * (lp + PW * q);
                const uint32_t* w = (const uint32_t*)(row + (size_t)(c < D ? c : 0) * IB);
#pragma unroll
                for (int h = 0; h < NW; ++h) raw[i][q][h] = w[h];
            }
        }
        auto val = [&](int i, int q, int h) -> float {  // channel 2p + h of token i
            if constexpr (IB == 4) return __uint_as_float(raw[i][q][h]);
            else return half_to_f32<DT>(h ? raw[i][q][0] >> 16 : raw[i][q][0]);
        };
        const PageRow pr = page_row(a.pages, e, b * G);
        uint32_t* meta = (uint32_t*)(a.meta + pr.base + e.meta[T] + (size_t)head * e.meta_hs[T]) + (size_t)(pr.row / G) * D;
        uint8_t* tile = smem + (size_t)wave * G * D;
#pragma unroll
        for (int q = 0; q < PPL; ++q) {
            const int c = 2 * (lp + PW * q);
            float mn[2], mx[2], sf[2], zf[2], rf[2];
            uint32_t sb[2], zb[2];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                mn[h] = INFINITY, mx[h] = -INFINITY;
#pragma unroll
                for (int i = 0; i < GL; ++i) mn[h] = fminf(mn[h], val(i, q, h)), mx[h] = fmaxf(mx[h], val(i, q, h));
                if constexpr (HS == 2) {  // the other half of the block: lane l ^ 32
                    mn[h] = fminf(mn[h], __shfl_xor(mn[h], 32));
                    mx[h] = fmaxf(mx[h], __shfl_xor(mx[h], 32));
                }
                sb[h] = f32_to_f16_bits((mx[h] - mn[h]) / L);
                zb[h] = f32_to_f16_bits(mn[h]);
                sf[h] = f16_to_f32(sb[h]);
                zf[h] = f16_to_f32(zb[h]);
                rf[h] = quant_rcp(sf[h]);
            }
            if (c < D) {
                if (t0 == 0) {
                    meta[c] = sb[0] | (zb[0] << 16);
                    meta[c + 1] = sb[1] | (zb[1] << 16);
                }
#pragma unroll
                for (int i = 0; i < GL; ++i)
                    *(uint16_t*)&tile[(t0 + i) * D + c] =
                        (uint16_t)(quant_code(val(i, q, 0), rf[0], sf[0], zf[0], L) | (quant_code(val(i, q, 1), rf[1], sf[1], zf[1], L) << 8));
            }
        }
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        uint8_t* codes = a.codes + pr.base + e.codes[T] + (size_t)head * e.codes_hs[T];
        for (int idx = lane; idx < G * UPR; idx += 64) {
            const int i = idx / UPR, u = idx - i * UPR;
            const uint4* src = (const uint4*)(tile + i * D + 32 * u);
            uint32_t cc[32];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const uint4 v4 = src[h];
                const uint32_t v[4] = {v4.x, v4.y, v4.z, v4.w};
#pragma unroll
                for (int m = 0; m < 4; ++m) {
                    cc[16 * h + 4 * m + 0] = v[m] & 0xffu;
                    cc[16 * h + 4 * m + 1] = (v[m] >> 8) & 0xffu;
                    cc[16 * h + 4 * m + 2] = (v[m] >> 16) & 0xffu;
                    cc[16 * h + 4 * m + 3] = v[m] >> 24;
                }
            }
            store_codes_rt(B, cc, (uint32_t*)(codes + (size_t)(pr.row + i) * (D * B / 8)) + u * B);
        }
    }
    if (k == 0)  // the first block's reads of the old residual rows are done (their values were used above)
        residual_rows<DT>(a, head, seq, b_end * G > len0 ? b_end * G : len0, len0, len1, 64);
}

// WIDE: the instantiation that also holds the wave path's larger tile (head_dim
// 256: two channel pairs per lane), which needs about twice the registers;
// launched only for appends that use it, so the others keep their occupancy.
// 64-token blocks at head_dim <= 64 split the block's tokens between the two
// halves of the wave (32 input words per lane, as for 32-token blocks).
template <int DT, bool WIDE>
__device__ __forceinline__ void channel_axis_any(const TensorArgs& a, int item, int head, int seq, uint32_t* smem) {
    if (!quant_wave_path(a.group, a.head_dim, a.in_dtype)) {
        channel_axis_part<DT>(a, item, head, seq, smem);
    } else if (a.group == 32 && a.head_dim <= 128) {
        channel_axis_wave<DT, 32, 1, 1>(a, item, head, seq, (uint8_t*)smem);
    } else if constexpr (In<DT>::bytes == 2) {
        if (a.group == 64) channel_axis_wave<DT, 64, 1, 2>(a, item, head, seq, (uint8_t*)smem);
        else if constexpr (WIDE) channel_axis_wave<DT, 32, 2, 1>(a, item, head, seq, (uint8_t*)smem);
    }
}

// One launch quantizes and appends both tensors: workgroups [0, gx_k) take the
// keys, [gx_k, gx_kv) the values, each with its own axis, and with a
// full-precision window [gx_kv, gridDim.x) copy the rows the window keeps.
// grid = (gx_kv + window workgroups, kv_heads, num_seqs x layers)
template <int DT, bool WIDE>
__global__ __launch_bounds__(kThreads) void quant_append_kernel(TensorArgs k0, TensorArgs v0, int gx_k, int gx_kv) {
    extern __shared__ uint32_t quant_smem[];
    int z = blockIdx.z, zv = blockIdx.z;
    const TensorArgs k = layer_args(k0, z, gridDim.z / k0.n_layers);
    const TensorArgs v = layer_args(v0, zv, gridDim.z / v0.n_layers);
    const int seq = z, head = blockIdx.y;
    uint32_t* smem = quant_smem;
    if ((int)blockIdx.x >= gx_kv) {
        window_rows<DT>(k, v, seq, head, (int)blockIdx.x - gx_kv, (int)gridDim.x - gx_kv, kThreads);
    } else if ((int)blockIdx.x < gx_k) {
        if (k.axis == 1) token_axis_part<DT>(k, blockIdx.x, head, seq);
        else channel_axis_any<DT, WIDE>(k, blockIdx.x, head, seq, smem);
    } else {
        const int item = (int)blockIdx.x - gx_k;
        if (v.axis == 1) token_axis_part<DT>(v, item, head, seq);
        else channel_axis_any<DT, WIDE>(v, item, head, seq, smem);
    }
}

// ---------------------------------------------------------------------------
// Decode attention, one split: workgroup = (chunk of C tokens, kv head, seq).
// Keys on the channel axis use the rewrite score_t = q.z_b + sum_c (q_c s_bc)
// code_tc, so each quantized key element costs one multiply-add; values on the
// token axis accumulate sum_t (p_t s_tg) code_tc plus sum_t p_t z_tg per group
// ([N] "Kuantisasi dapat memindahkan pekerjaan ke decode path": unpacking and
// scale application inside the attention kernel). Query heads sharing the kv
// head are processed one after the other. Each split writes (m, l, o) in the
// log2 domain for the merge.
// ---------------------------------------------------------------------------

// acc += sum_j q[j] * code_j over one unit.
template <int B>
__device__ __forceinline__ float dot_unit(const uint32_t* unit, const float* q, float acc) {
    uint32_t w[B];
    load_unit<B>(unit, w);
#pragma unroll
    for (int j = 0; j < 32; ++j) acc = fmaf(q[j], (float)code_at<B>(w, j), acc);
    return acc;
}

template <int B>
__device__ __forceinline__ void axpy_unit(const uint32_t* unit, float wgt, float (&acc)[32]) {
    uint32_t w[B];
    load_unit<B>(unit, w);
#pragma unroll
    for (int j = 0; j < 32; ++j) acc[j] = fmaf(wgt, (float)code_at<B>(w, j), acc[j]);
}

template <int BK>
__device__ __forceinline__ float key_score_channel(const uint32_t* row, const float* qb, int UPR, float acc) {
    for (int u = 0; u < UPR; ++u) acc = dot_unit<BK>(row + u * BK, qb + 32 * u, acc);
    return acc;
}

template <int BK>
__device__ __forceinline__ float key_score_token(const uint32_t* row, const uint32_t* meta_row, const float* qr,
                                                 const float* qsum, int UPR, int UG) {
    float acc = 0.f;
    for (int g = 0; g < UPR / UG; ++g) {
        float part = 0.f;
        for (int u = g * UG; u < (g + 1) * UG; ++u) part = dot_unit<BK>(row + u * BK, qr + 32 * u, part);
        const uint32_t w = meta_row[g];
        acc = fmaf(f16_to_f32(w), part, acc);
        acc = fmaf(f16_to_f32(w >> 16), qsum[g], acc);
    }
    return acc;
}

// vc, vm: head 0 offsets of the value codes and metadata inside a page (pool
// offsets with contiguous storage); token t is found through the page list.
template <int BV>
__device__ __forceinline__ void value_pass(const uint32_t* pages, const SeqEntry& e, const uint8_t* vc,
                                           const uint8_t* vm, const float* sc, int t0, int t1, int tl, int TL, int u,
                                           int D, int Gv, float (&acc)[32], float& zacc) {
    const int g = (32 * u) / Gv, gpr = D / Gv;
    for (int t = t0 + tl; t < t1; t += TL) {
        const float p = sc[t - t0];
        const PageRow pr = page_row(pages, e, t);
        const uint32_t w = ((const uint32_t*)(vm + pr.base))[(size_t)pr.row * gpr + g];
        zacc = fmaf(p, f16_to_f32(w >> 16), zacc);
        const uint32_t* unit = (const uint32_t*)(vc + pr.base + (size_t)pr.row * (D * BV / 8)) + u * BV;
        axpy_unit<BV>(unit, p * f16_to_f32(w), acc);
    }
}

// Values grouped along tokens like keys (one step and zero per channel per
// block of G tokens): x_hat = fma(code, s_bc, z_bc) per element, added with
// weight p; tokens past the last whole block are read from the residual rows
// vr (row t mod G, input dtype). nqv: tokens with quantized values.
template <int DT, int BV>
__device__ __forceinline__ void value_pass_channel(const uint32_t* pages, const SeqEntry& e, const uint8_t* vc,
                                                   const uint8_t* vm, const uint8_t* vr, const float* sc, int t0,
                                                   int t1, int nqv, int tl, int TL, int u, int D, int Gv,
                                                   float (&acc)[32]) {
    for (int t = t0 + tl; t < t1; t += TL) {
        const float p = sc[t - t0];
        if (t < nqv) {
            const PageRow pr = page_row(pages, e, t);
            uint32_t w[BV];
            load_unit<BV>((const uint32_t*)(vc + pr.base + (size_t)pr.row * (D * BV / 8)) + u * BV, w);
            const uint32_t* meta = (const uint32_t*)(vm + pr.base) + (size_t)(pr.row / Gv) * D + 32 * u;
#pragma unroll
            for (int j = 0; j < 32; ++j) {
                const uint32_t m = meta[j];
                acc[j] = fmaf(p, fmaf((float)code_at<BV>(w, j), f16_to_f32(m), f16_to_f32(m >> 16)), acc[j]);
            }
        } else {
            const uint8_t* row = vr + (size_t)(t % Gv) * D * In<DT>::bytes;
#pragma unroll
            for (int j = 0; j < 32; ++j) acc[j] = fmaf(p, load_in<DT>(row, 32 * u + j), acc[j]);
        }
    }
}

template <int B>
__device__ __forceinline__ uint32_t code_of(const uint32_t* row, int ch) {
    const uint32_t* unit = row + (ch >> 5) * B;
    const int pos = (ch & 31) * B, wi = pos >> 5, sh = pos & 31;
    uint32_t v = unit[wi] >> sh;
    if (sh + B > 32) v |= unit[wi + 1] << (32 - sh);
    return v & ((1u << B) - 1u);
}

// Score of token t: the key reconstructed per channel (fma(code, s, z), block
// metadata bm[D]) or read from the residual row `rrow` (input dtype), rotated to
// position t pair by pair (i, i + D/2), dotted with the query q.
template <int DT, int BK>
__device__ float rope_score(const uint32_t* row, const uint32_t* bm, const uint8_t* rrow, const float* q,
                            const double* th, int D, int t) {
    const int h = D >> 1;
    float acc = 0.f;
    for (int i = 0; i < h; ++i) {
        float xa, xb;
        if (row) {
            const uint32_t ma = bm[i], mb = bm[i + h];
            xa = fmaf((float)code_of<BK>(row, i), f16_to_f32(ma), f16_to_f32(ma >> 16));
            xb = fmaf((float)code_of<BK>(row, i + h), f16_to_f32(mb), f16_to_f32(mb >> 16));
        } else {
            xa = load_in<DT>(rrow, i);
            xb = load_in<DT>(rrow, i + h);
        }
        float c, s;
        rope_cs(t, th[i], c, s);
        acc = fmaf(q[i], xa * c - xb * s, acc);
        acc = fmaf(q[i + h], xa * s + xb * c, acc);
    }
    return acc;
}

template <int DT>
__global__ __launch_bounds__(kThreads) void decode_split_kernel(DecodeArgs a0) {
    extern __shared__ float smem[];
    int z = blockIdx.z;
    const DecodeArgs a = layer_args(a0, z, gridDim.z / a0.n_layers);
    const int seq = z, kvh = blockIdx.y, chunk = blockIdx.x;
    const int len = a.len[seq];
    int tb, te;  // quantized tokens: all, or the whole key blocks inside [sinks, len - window)
    quant_range(a, len, tb, te);
    const int C = a.chunk, t0 = tb + chunk * C;
    if (t0 >= te) return;
    const int t1 = min(t0 + C, te), nt = t1 - t0;
    const int D = a.head_dim, UPR = D >> 5, R = a.q_heads / a.kv_heads;
    const int Gk = a.group_k, Gv = a.group_v;
    const bool kch = a.axis_k == 0;
    const SeqEntry& e = a.table[seq];
    const int BK = e.bits[0], BV = e.bits[1];
    const int nqk = a.win_mode ? te : kch ? (len / Gk) * Gk : len;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
    constexpr int IB = In<DT>::bytes;

    // LDS carve-up (floats): q[R][D] | scores[C] | qk[8][256] | small[64] | red[256*32]
    float* q_s = smem;
    float* sc = q_s + R * D;
    float* qk = sc + C;
    float* small = qk + 8 * 256;  // [0,8) bias, [8,16) qsum, [16,20) reduction scratch
    float* red = small + 64;
    double* th = (double*)(red + 256 * 32);  // rotary frequencies [D/2] (rope_base > 0)
    const bool rope = a.rope_base > 0.0;

    // head kvh's codes and metadata inside a page (pool offsets with contiguous storage)
    const uint8_t* kc = a.codes + e.codes[0] + (size_t)kvh * e.codes_hs[0];
    const uint8_t* kmp = a.meta + e.meta[0] + (size_t)kvh * e.meta_hs[0];
    const uint8_t* kr = a.resid + e.resid[0] + (size_t)kvh * e.resid_hs[0];
    const uint8_t* vc = a.codes + e.codes[1] + (size_t)kvh * e.codes_hs[1];
    const uint8_t* vm = a.meta + e.meta[1] + (size_t)kvh * e.meta_hs[1];
    const uint8_t* vr = a.resid + e.resid[1] + (size_t)kvh * e.resid_hs[1];  // per-channel values' residual rows
    // key code row of token t; key metadata of channel-axis block b (D words)
    // or of token t (D / G words)
    auto krow = [&](int t) -> const uint32_t* {
        const PageRow pr = page_row(a.pages, e, t);
        return (const uint32_t*)(kc + pr.base + (size_t)pr.row * (D * BK / 8));
    };
    auto kmeta_block = [&](int b) -> const uint32_t* {
        const PageRow pr = page_row(a.pages, e, b * Gk);
        return (const uint32_t*)(kmp + pr.base) + (size_t)(pr.row / Gk) * D;
    };
    auto kmeta_token = [&](int t) -> const uint32_t* {
        const PageRow pr = page_row(a.pages, e, t);
        return (const uint32_t*)(kmp + pr.base) + (size_t)pr.row * (D / Gk);
    };

    for (int i = tid; i < R * D; i += kThreads) {
        const int r = i / D, ch = i % D;
        q_s[i] = load_in<DT>(a.q, ((size_t)seq * a.q_heads + kvh * R + r) * D + ch) * a.qscale;
    }
    if (rope)
        for (int i = tid; i < D / 2; i += kThreads) th[i] = pow(a.rope_base, -2.0 * i / D);
    __syncthreads();

    for (int r = 0; r < R; ++r) {
        const float* qr = q_s + r * D;
        const int hq = kvh * R + r;
        // ---- keys -------------------------------------------------------
        if (kch && rope) {
            // one thread per token: reconstruct, rotate to the token's position, score
            for (int t = t0 + tid; t < t1; t += kThreads) {
                const bool quant = t < nqk;
                const uint32_t* row = quant ? krow(t) : nullptr;
                const uint32_t* bm = quant ? kmeta_block(t / Gk) : nullptr;
                const uint8_t* rrow = kr + (size_t)(t % Gk) * D * IB;
                float acc;
                switch (BK) {
                    case 2: acc = rope_score<DT, 2>(row, bm, rrow, qr, th, D, t); break;
                    case 3: acc = rope_score<DT, 3>(row, bm, rrow, qr, th, D, t); break;
                    case 4: acc = rope_score<DT, 4>(row, bm, rrow, qr, th, D, t); break;
                    case 6: acc = rope_score<DT, 6>(row, bm, rrow, qr, th, D, t); break;
                    default: acc = rope_score<DT, 8>(row, bm, rrow, qr, th, D, t); break;
                }
                sc[t - t0] = acc;
            }
        } else if (kch) {
            const int kend = min(t1, nqk);
            for (int tile0 = t0; tile0 < kend; tile0 += kThreads) {
                const int tile_end = min(tile0 + kThreads, kend);
                const int b0 = tile0 / Gk;
                const int nbl = (tile_end - tile0 + Gk - 1) / Gk;
                for (int idx = tid; idx < nbl * D; idx += kThreads) {
                    const int bl = idx / D, ch = idx % D;
                    qk[idx] = qr[ch] * f16_to_f32(kmeta_block(b0 + bl)[ch]);
                }
                for (int bl = wave; bl < nbl; bl += 4) {
                    float p = 0.f;
                    const uint32_t* bm = kmeta_block(b0 + bl);
                    for (int ch = lane; ch < D; ch += 64) p = fmaf(qr[ch], f16_to_f32(bm[ch] >> 16), p);
                    p = wave_sum(p);
                    if (lane == 0) small[bl] = p;
                }
                __syncthreads();
                const int t = tile0 + tid;
                if (t < tile_end) {
                    const int bl = t / Gk - b0;
                    const uint32_t* row = krow(t);
                    float acc = small[bl];
                    const float* qb = qk + bl * D;
                    switch (BK) {
                        case 2: acc = key_score_channel<2>(row, qb, UPR, acc); break;
                        case 3: acc = key_score_channel<3>(row, qb, UPR, acc); break;
                        case 4: acc = key_score_channel<4>(row, qb, UPR, acc); break;
                        case 6: acc = key_score_channel<6>(row, qb, UPR, acc); break;
                        default: acc = key_score_channel<8>(row, qb, UPR, acc); break;
                    }
                    sc[t - t0] = acc;
                }
                __syncthreads();
            }
            // residual key rows (input dtype)
            const int rs = max(t0, nqk);
            for (int t = rs + tid; t < t1; t += kThreads) {
                const uint8_t* rrow = kr + (size_t)(t % Gk) * D * IB;
                float acc = 0.f;
                for (int ch = 0; ch < D; ++ch) acc = fmaf(qr[ch], load_in<DT>(rrow, ch), acc);
                sc[t - t0] = acc;
            }
        } else {
            const int UG = Gk >> 5;
            if (tid < D / Gk) {
                float s = 0.f;
                for (int ch = tid * Gk; ch < (tid + 1) * Gk; ++ch) s += qr[ch];
                small[8 + tid] = s;
            }
            __syncthreads();
            for (int t = t0 + tid; t < t1; t += kThreads) {
                const uint32_t* row = krow(t);
                const uint32_t* mrow = kmeta_token(t);
                float acc;
                switch (BK) {
                    case 2: acc = key_score_token<2>(row, mrow, qr, small + 8, UPR, UG); break;
                    case 3: acc = key_score_token<3>(row, mrow, qr, small + 8, UPR, UG); break;
                    case 4: acc = key_score_token<4>(row, mrow, qr, small + 8, UPR, UG); break;
                    case 6: acc = key_score_token<6>(row, mrow, qr, small + 8, UPR, UG); break;
                    default: acc = key_score_token<8>(row, mrow, qr, small + 8, UPR, UG); break;
                }
                sc[t - t0] = acc;
            }
        }
        __syncthreads();
        // ---- softmax over this split ------------------------------------
        float m = -INFINITY;
        for (int i = tid; i < nt; i += kThreads) m = fmaxf(m, sc[i]);
        m = block_max(m, small + 16);
        float l = 0.f;
        for (int i = tid; i < nt; i += kThreads) {
            const float p = exp2f(sc[i] - m);
            sc[i] = p;
            l += p;
        }
        l = block_sum(l, small + 16);  // its barriers also publish sc
        // ---- values -----------------------------------------------------
        const int TL = kThreads / UPR, tl = tid / UPR, u = tid % UPR;
        float acc[32];
#pragma unroll
        for (int j = 0; j < 32; ++j) acc[j] = 0.f;
        float zacc = 0.f;
        if (a.axis_v == 0) {  // per-channel values (windowed tokens all lie in whole blocks)
            const int nqv = a.win_mode ? te : (len / Gv) * Gv;
            switch (BV) {
                case 2: value_pass_channel<DT, 2>(a.pages, e, vc, vm, vr, sc, t0, t1, nqv, tl, TL, u, D, Gv, acc); break;
                case 3: value_pass_channel<DT, 3>(a.pages, e, vc, vm, vr, sc, t0, t1, nqv, tl, TL, u, D, Gv, acc); break;
                case 4: value_pass_channel<DT, 4>(a.pages, e, vc, vm, vr, sc, t0, t1, nqv, tl, TL, u, D, Gv, acc); break;
                case 6: value_pass_channel<DT, 6>(a.pages, e, vc, vm, vr, sc, t0, t1, nqv, tl, TL, u, D, Gv, acc); break;
                default: value_pass_channel<DT, 8>(a.pages, e, vc, vm, vr, sc, t0, t1, nqv, tl, TL, u, D, Gv, acc); break;
            }
        } else {
            switch (BV) {
                case 2: value_pass<2>(a.pages, e, vc, vm, sc, t0, t1, tl, TL, u, D, Gv, acc, zacc); break;
                case 3: value_pass<3>(a.pages, e, vc, vm, sc, t0, t1, tl, TL, u, D, Gv, acc, zacc); break;
                case 4: value_pass<4>(a.pages, e, vc, vm, sc, t0, t1, tl, TL, u, D, Gv, acc, zacc); break;
                case 6: value_pass<6>(a.pages, e, vc, vm, sc, t0, t1, tl, TL, u, D, Gv, acc, zacc); break;
                default: value_pass<8>(a.pages, e, vc, vm, sc, t0, t1, tl, TL, u, D, Gv, acc, zacc); break;
            }
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) red[tl * D + 32 * u + j] = acc[j] + zacc;
        __syncthreads();
        const size_t slot = ((size_t)seq * a.q_heads + hq) * a.max_chunks + chunk;
        for (int ch = tid; ch < D; ch += kThreads) {
            float o = 0.f;
            for (int i = 0; i < TL; ++i) o += red[i * D + ch];
            a.ws_o[slot * D + ch] = o;
        }
        if (tid == 0) {
            a.ws_ml[slot * 2 + 0] = m;
            a.ws_ml[slot * 2 + 1] = l;
        }
        __syncthreads();  // red, sc and small are reused by the next query head
    }
}

// Merge the splits of one (seq, q head): m* = max m_i, l* = sum l_i 2^(m_i - m*),
// out = sum o_i 2^(m_i - m*) / l*. A sequence of length 0 gets zeros.
__global__ __launch_bounds__(kThreads) void merge_kernel(DecodeArgs a0) {
    // grid = (q_heads x ceil(D / 64), num_seqs x layers): one workgroup per
    // (seq, query head, 64-channel slice). Every wave computes the same maximum
    // and denominator over the splits (lane-strided, then wave reductions);
    // wave w sums the splits w, w + 4, ... of channel slice + lane, and the four
    // partial sums are added in a fixed order.
    __shared__ float part[kThreads];
    int y = blockIdx.y;
    const DecodeArgs a = layer_args(a0, y, gridDim.y / a0.n_layers);
    const int D = a.head_dim, nsl = (D + 63) >> 6;
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int hq = blockIdx.x / nsl, c = (blockIdx.x - hq * nsl) * 64 + lane, seq = y;
    const int len = a.len[seq];
    float* out = a.out + ((size_t)seq * a.q_heads + hq) * D;
    int nch;
    if (a.win_mode && a.split_floor) {
        // single-query kernel: max(1, (te - tb) / chunk) splits, the last of
        // which also read the full-precision rows; one split was written directly
        int tb, te;
        quant_range(a, len, tb, te);
        nch = max(1, (te - tb) / a.chunk);
        if (len == 0 || nch <= 1) return;
    } else if (a.win_mode) {
        // quantized splits, then the full-precision rows' splits
        int tb, te;
        quant_range(a, len, tb, te);
        nch = len == 0 ? 0 : quant_splits(a, tb, te) + (fp_count(a, len, te) + kWinTokens - 1) / kWinTokens;
    } else {
        // single-query kernel: max(1, len / chunk) splits; one split was written directly
        if (a.split_floor && len / a.chunk <= 1) return;
        nch = a.split_floor ? len / a.chunk : (len + a.chunk - 1) / a.chunk;
    }
    if (nch == 0) {
        if (wave == 0 && c < D) out[c] = 0.f;
        return;
    }
    const size_t base = ((size_t)seq * a.q_heads + hq) * a.max_chunks;
    const float* ml = a.ws_ml + base * 2;
    float M = -INFINITY;
    for (int i = lane; i < nch; i += 64) M = fmaxf(M, ml[2 * i]);
    M = wave_max(M);
    float L = 0.f;
    for (int i = lane; i < nch; i += 64) L += ml[2 * i + 1] * exp2f(ml[2 * i] - M);
    L = wave_sum(L);
    const float* src = a.ws_o + base * D;
    const int cc = min(c, D - 1);
    float o = 0.f;
    // 8 of the wave's splits in flight at a time (clamped indices, zero weights past the end)
    for (int i0 = wave; i0 < nch; i0 += 32) {
        float v[8], wgt[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            const int i = min(i0 + 4 * k, nch - 1);
            v[k] = src[(size_t)i * D + cc];
            wgt[k] = i0 + 4 * k < nch ? exp2f(ml[2 * i] - M) : 0.f;
        }
#pragma unroll
        for (int k = 0; k < 8; ++k) o = fmaf(v[k], wgt[k], o);
    }
    part[threadIdx.x] = o;
    __syncthreads();
    if (wave == 0 && c < D) out[c] = (((part[lane] + part[64 + lane]) + part[128 + lane]) + part[192 + lane]) * (1.0f / L);
}

// ---------------------------------------------------------------------------
// Full-precision window and sinks ([U] "O Imposto dos Sistemas ...": recent
// tokens in full precision; [U] "Onde o Trabalho Esta Indo": sink tokens too).
// Workgroup = (split of kWinTokens full-precision tokens, (kv head, group of up
// to kWinHeads of its query heads), seq): the attention partial (m, l, o) of
// each of those query heads over its
// tokens, read from the window area in the input dtype, written as split
// nq + blockIdx.x (after the quantized kernel's nq splits). Scores: thread =
// (token, quarter of the channels) with its inputs in registers; values:
// thread = (token part, channel) with its tokens' inputs in registers; one
// query head at a time against them.
// LDS: q [R][D] | weights [R][kWinTokens] | per-head m, l | [kThreads] reduction.
// ---------------------------------------------------------------------------
// 8 consecutive input elements at element offset `off` (16-byte aligned for
// 2-byte inputs, 32-byte for float32) as floats.
template <int DT>
__device__ __forceinline__ void load8(const uint8_t* base, size_t off, float (&x)[8]) {
    if constexpr (DT == 0) {
        const uint4* p = (const uint4*)((const float*)base + off);
        const uint4 a = p[0], b = p[1];
        const uint32_t w[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
        for (int j = 0; j < 8; ++j) x[j] = __uint_as_float(w[j]);
    } else {
        const uint4 a = *(const uint4*)((const uint16_t*)base + off);
        const uint32_t w[4] = {a.x, a.y, a.z, a.w};
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            x[2 * j] = half_to_f32<DT>(w[j]);
            x[2 * j + 1] = half_to_f32<DT>(w[j] >> 16);
        }
    }
}

template <int DT, int D>
__global__ __launch_bounds__(kThreads) void decode_window_kernel(DecodeArgs a0) {
    extern __shared__ float win_smem[];
    constexpr int DQ = D / 4;          // channels per thread in the score phase
    constexpr int TP = kThreads / D;   // token parts in the value phase
    constexpr int TPT = kWinTokens / TP;  // tokens per thread in the value phase
    constexpr int QPT = (kWinHeads * D + kThreads - 1) / kThreads;  // query elements per thread, at most
    int z = blockIdx.z;
    const DecodeArgs a = layer_args(a0, z, gridDim.z / a0.n_layers);
    // y = (kv head, group of up to kWinHeads of its query heads)
    const int RA = a.q_heads / a.kv_heads, HG = (RA + kWinHeads - 1) / kWinHeads;
    const int seq = z, kvh = blockIdx.y / HG, h0 = (blockIdx.y % HG) * kWinHeads;
    const int R = min(kWinHeads, RA - h0);  // query heads of this workgroup: h0 .. h0 + R - 1
    const int len = a.len[seq];
    int tb, te;
    quant_range(a, len, tb, te);
    const int nfp = fp_count(a, len, te);
    const int i0 = blockIdx.x * kWinTokens;
    if (len == 0 || i0 >= nfp) return;
    const int n = min(kWinTokens, nfp - i0);
    const int nq = quant_splits(a, tb, te);
    const int tid = threadIdx.x;
    const SeqEntry& e = a.table[seq];
    const uint8_t* kw = a.resid + e.resid[0] + (size_t)kvh * e.resid_hs[0] + a.win_off[0];
    const uint8_t* vw = a.resid + e.resid[1] + (size_t)kvh * e.resid_hs[1] + a.win_off[1];
    float* q_s = win_smem;                 // [R][D], scaled to the log2 domain
    float* p_s = q_s + R * D;              // [R][kWinTokens]: scores, then weights
    float* ml_s = p_s + R * kWinTokens;    // [R][2]
    float* red = ml_s + 2 * R;             // [TP][R][D] partial outputs (TP > 1)
    int* row_s = (int*)(red + (TP > 1 ? TP * R * D : 0));  // [kWinTokens]: window row of each token
    int* pos_s = row_s + kWinTokens;                      // [kWinTokens]: position of each token
    double* th = (double*)(((uintptr_t)(pos_s + kWinTokens) + 7) & ~(uintptr_t)7);  // rotary frequencies [D/2]
    const bool rope = a.rope_base > 0.0;
    if (rope)
        for (int i = tid; i < D / 2; i += kThreads) th[i] = pow(a.rope_base, -2.0 * i / D);
    {
        // the R query rows: every load issued before the first use. Loads are
        // unconditional, from clamped (valid) addresses: a load under a branch
        // is followed by its own wait, which would serialize them.
        const size_t qo = ((size_t)seq * a.q_heads + (size_t)kvh * RA + h0) * D;
        float qv[QPT];
#pragma unroll
        for (int k = 0; k < QPT; ++k) qv[k] = load_in<DT>(a.q, qo + min(tid + k * kThreads, R * D - 1));
#pragma unroll
        for (int k = 0; k < QPT; ++k) {
            const int i = tid + k * kThreads;
            if (i < R * D) q_s[i] = qv[k] * a.qscale;
        }
    }
    if (tid < kWinTokens) {
        const int t = tid < n ? fp_token(a, len, te, i0 + tid) : 0;
        row_s[tid] = tid < n ? window_row(t, a.sinks, a.win_rows, e.ring) : 0;
        pos_s[tid] = t;
    }
    __syncthreads();

    // ---- scores: thread = (token i, channel quarter p); the quarter's inputs come
    // in 16-byte loads issued up front, the 16 query heads' sums stay in registers
    {
        const int i = tid >> 2, p = tid & 3;
        float x[DQ];
        const size_t base = (size_t)row_s[i] * D + p * DQ;
        // (row_s is 0 past n: a valid row, whose contents are discarded)
#pragma unroll
        for (int j = 0; j < DQ; j += 8) {
            float y[8];
            load8<DT>(kw, base + j, y);
#pragma unroll
            for (int u = 0; u < 8; ++u) x[j + u] = i < n ? y[u] : 0.f;
        }
        if (rope) {
            // keys cached before the rotary embedding: rotate to the token's
            // position; channel pair (c, c + D/2) is split between quarters p
            // and p ^ 2 of the same token (threads tid and tid ^ 2)
            const int t = pos_s[i];
#pragma unroll
            for (int j = 0; j < DQ; ++j) {
                const float other = __shfl_xor(x[j], 2);
                const int pair = (p & 1) * DQ + j;
                float c, sn;
                rope_cs(t, th[pair], c, sn);
                x[j] = p < 2 ? x[j] * c - other * sn : other * sn + x[j] * c;
            }
        }
        // one query head per iteration, not unrolled: the code stays small
        // (it runs once per workgroup, so its instruction fetches are cold)
#pragma unroll 1
        for (int r = 0; r < R; ++r) {
            const float* qr = q_s + r * D + p * DQ;
            float v = 0.f;
#pragma unroll
            for (int j = 0; j < DQ; ++j) v = fmaf(qr[j], x[j], v);
            v += __shfl_xor(v, 1);
            v += __shfl_xor(v, 2);
            if (p == 0) p_s[r * kWinTokens + i] = i < n ? v : -INFINITY;
        }
    }
    __syncthreads();
    // ---- softmax of this split per query head: wave w takes heads w, w + 4, ...
    {
        const int wave = tid >> 6, lane = tid & 63;
        for (int r = wave; r < R; r += kThreads / 64) {
            const float sc = p_s[r * kWinTokens + lane];
            const float m = wave_max(sc);
            const float w = lane < n ? exp2f(sc - m) : 0.f;
            p_s[r * kWinTokens + lane] = w;
            const float l = wave_sum(w);
            if (lane == 0) {
                ml_s[2 * r] = m;
                ml_s[2 * r + 1] = l;
            }
        }
    }
    __syncthreads();
    // ---- values: thread = (token part tp, channel c); its tokens' inputs are
    // loaded up front and one query head at a time is applied. Threads past TP * D
    // (when D does not divide kThreads) only join the barriers; rows past n may
    // never have been written, so they are not read.
    const int tp = tid / D, c = tid % D;
    const bool active = tp < TP;
    const int tpc = active ? tp : 0;  // clamped: every load is unconditional and in bounds
    float v[TPT];
#pragma unroll
    for (int k = 0; k < TPT; ++k) v[k] = load_in<DT>(vw, (size_t)row_s[tpc + k * TP] * D + c);
#pragma unroll
    for (int k = 0; k < TPT; ++k) v[k] = active && tp + k * TP < n ? v[k] : 0.f;
    const int slot0 = nq + blockIdx.x;
    const size_t slot_base = ((size_t)seq * a.q_heads + (size_t)kvh * RA + h0) * a.max_chunks + slot0;
    if constexpr (TP > 1) {
        if (active) {
#pragma unroll 1
            for (int r = 0; r < R; ++r) {
                float o = 0.f;
#pragma unroll
                for (int k = 0; k < TPT; ++k) o = fmaf(p_s[r * kWinTokens + tp + k * TP], v[k], o);
                red[(tp * R + r) * D + c] = o;
            }
        }
        __syncthreads();
        for (int i = tid; i < R * D; i += kThreads) {
            const int r = i / D, ch = i % D;
            float sum = 0.f;
#pragma unroll
            for (int k = 0; k < TP; ++k) sum += red[(k * R + r) * D + ch];
            a.ws_o[(slot_base + (size_t)r * a.max_chunks) * D + ch] = sum * a.ws_scale;
        }
    } else if (active) {
#pragma unroll 1
        for (int r = 0; r < R; ++r) {
            float o = 0.f;
#pragma unroll
            for (int k = 0; k < TPT; ++k) o = fmaf(p_s[r * kWinTokens + tp + k * TP], v[k], o);
            a.ws_o[(slot_base + (size_t)r * a.max_chunks) * D + c] = o * a.ws_scale;
        }
    }
    if (tid < R) {
        a.ws_ml[(slot_base + (size_t)tid * a.max_chunks) * 2 + 0] = ml_s[2 * tid];
        a.ws_ml[(slot_base + (size_t)tid * a.max_chunks) * 2 + 1] = ml_s[2 * tid + 1] * a.ws_scale;
    }
}

// ---------------------------------------------------------------------------
// Dequantize one tensor of one sequence into float32 [Hkv][len][D]:
// x_hat = fma(code, s, z), which is the correctly rounded value of the exact
// z + code * s ([N] "Kuantisasi dapat memindahkan pekerjaan ke decode path":
// the unfused alternative); residual rows are converted exactly.
// grid = (ceil(len * D/32 / 256), kv_heads)
// ---------------------------------------------------------------------------
template <int B>
__device__ __forceinline__ void dequant_unit(const uint32_t* unit, const uint32_t* meta, bool per_channel, float* out) {
    uint32_t w[B];
    load_unit<B>(unit, w);
    if (per_channel) {
#pragma unroll
        for (int j = 0; j < 32; ++j) {
            const uint32_t m = meta[j];
            out[j] = fmaf((float)code_at<B>(w, j), f16_to_f32(m), f16_to_f32(m >> 16));
        }
    } else {
        const uint32_t m = meta[0];
        const float s = f16_to_f32(m), z = f16_to_f32(m >> 16);
#pragma unroll
        for (int j = 0; j < 32; ++j) out[j] = fmaf((float)code_at<B>(w, j), s, z);
    }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void dequant_kernel(DequantArgs a) {
    const int D = a.head_dim, UPR = D >> 5;
    const int idx = blockIdx.x * kThreads + threadIdx.x;
    const int t = idx / UPR, u = idx % UPR, head = blockIdx.y;
    if (t >= a.len) return;
    const int T = a.tensor, B = a.entry.bits[T], G = a.group;
    const bool ch = a.axis == 0;
    const int nq = ch ? (a.len / G) * G : a.len;
    float* out = a.out + ((size_t)head * a.len + t) * D + 32 * u;
    if (a.win_mode) {
        // the full-precision tokens of the window and the sinks, as the attention reads them
        const int r = a.len - a.window;
        const int q = max(r > 0 ? r / a.tblock * a.tblock : 0, a.sinks);
        if (t < a.sinks || t >= q) {
            const uint8_t* wrow = a.resid + a.entry.resid[T] + (size_t)head * a.entry.resid_hs[T] + a.win_off +
                                  (size_t)window_row(t, a.sinks, a.win_rows, a.entry.ring) * D * In<DT>::bytes;
            for (int j = 0; j < 32; ++j) out[j] = load_in<DT>(wrow, 32 * u + j);
            return;
        }
    }
    if (t < nq) {
        const PageRow pr = page_row(a.pages, a.entry, t);
        const uint32_t* unit = (const uint32_t*)(a.codes + pr.base + a.entry.codes[T] +
                                                 (size_t)head * a.entry.codes_hs[T] + (size_t)pr.row * (D * B / 8)) +
                               u * B;
        const uint32_t* meta =
            (const uint32_t*)(a.meta + pr.base + a.entry.meta[T] + (size_t)head * a.entry.meta_hs[T]);
        meta += ch ? (size_t)(pr.row / G) * D + 32 * u : (size_t)pr.row * (D / G) + (32 * u) / G;
        float v[32];
        switch (B) {
            case 2: dequant_unit<2>(unit, meta, ch, v); break;
            case 3: dequant_unit<3>(unit, meta, ch, v); break;
            case 4: dequant_unit<4>(unit, meta, ch, v); break;
            case 6: dequant_unit<6>(unit, meta, ch, v); break;
            default: dequant_unit<8>(unit, meta, ch, v); break;
        }
#pragma unroll
        for (int j = 0; j < 32; ++j) out[j] = v[j];
    } else {
        const uint8_t* rrow = a.resid + a.entry.resid[T] + (size_t)head * a.entry.resid_hs[T] +
                              (size_t)(t % G) * D * In<DT>::bytes;
        for (int j = 0; j < 32; ++j) out[j] = load_in<DT>(rrow, 32 * u + j);
    }
}

}  // namespace

// ---------------------------------------------------------------------------
// Launchers
// ---------------------------------------------------------------------------

size_t decode_lds_bytes(int R, int D, int C) {
    return sizeof(float) * ((size_t)R * D + C + 8 * 256 + 64 + 256 * 32) + sizeof(double) * kMaxHeadDim / 2;
}

hipError_t launch_quant_append(const TensorArgs& k, const TensorArgs& v, int gx_k, int gx_v, int max_new, hipStream_t s) {
    int gx_w = 0;  // window copy: enough workgroups for the rows kept, at most 64
    if (k.win_mode) {
        const long elems = (long)std::min(max_new, k.sinks + k.win_rows) * k.head_dim;
        gx_w = (int)std::min<long>(std::max<long>(1, (elems + kThreads - 1) / kThreads), 64);
    }
    const int gx_kv = gx_k + gx_v;
    dim3 grid(gx_kv + gx_w, k.kv_heads, k.num_seqs * k.n_layers);
    size_t lds = 0;
    for (const TensorArgs* t : {&k, &v})
        if (t->axis == 0)
            lds = std::max(lds, quant_wave_path(t->group, t->head_dim, t->in_dtype)
                                    ? (size_t)kQuantBlocksPerGroup * t->group * t->head_dim
                                    : std::max((size_t)t->group * t->head_dim, (size_t)2 * 2 * kThreads * sizeof(float)));
    bool wide = false;
    for (const TensorArgs* t : {&k, &v})
        wide |= t->axis == 0 && quant_wave_path(t->group, t->head_dim, t->in_dtype) && quant_wave_wide(t->group, t->head_dim);
    switch (k.in_dtype) {
        case 0: hipLaunchKernelGGL((quant_append_kernel<0, false>), grid, dim3(kThreads), lds, s, k, v, gx_k, gx_kv); break;
        case 1:
            if (wide) hipLaunchKernelGGL((quant_append_kernel<1, true>), grid, dim3(kThreads), lds, s, k, v, gx_k, gx_kv);
            else hipLaunchKernelGGL((quant_append_kernel<1, false>), grid, dim3(kThreads), lds, s, k, v, gx_k, gx_kv);
            break;
        default:
            if (wide) hipLaunchKernelGGL((quant_append_kernel<2, true>), grid, dim3(kThreads), lds, s, k, v, gx_k, gx_kv);
            else hipLaunchKernelGGL((quant_append_kernel<2, false>), grid, dim3(kThreads), lds, s, k, v, gx_k, gx_kv);
            break;
    }
    return hipGetLastError();
}

hipError_t launch_merge(const DecodeArgs& a, hipStream_t s) {
    hipLaunchKernelGGL(merge_kernel, dim3(a.q_heads * ((a.head_dim + 63) / 64), a.num_seqs * a.n_layers),
                       dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

hipError_t launch_decode(const DecodeArgs& a, hipStream_t s) {
    const int R = a.q_heads / a.kv_heads;
    dim3 grid(a.max_chunks - a.win_splits, a.kv_heads, a.num_seqs * a.n_layers);  // quantized splits only
    const size_t lds = decode_lds_bytes(R, a.head_dim, a.chunk);
    switch (a.in_dtype) {
        case 0: hipLaunchKernelGGL(decode_split_kernel<0>, grid, dim3(kThreads), lds, s, a); break;
        case 1: hipLaunchKernelGGL(decode_split_kernel<1>, grid, dim3(kThreads), lds, s, a); break;
        default: hipLaunchKernelGGL(decode_split_kernel<2>, grid, dim3(kThreads), lds, s, a); break;
    }
    return hipGetLastError();  // the caller launches the split merge
}

template <int DT>
void window_d(const DecodeArgs& a, dim3 grid, size_t lds, hipStream_t s) {
    switch (a.head_dim) {
        case 32: hipLaunchKernelGGL((decode_window_kernel<DT, 32>), grid, dim3(kThreads), lds, s, a); break;
        case 64: hipLaunchKernelGGL((decode_window_kernel<DT, 64>), grid, dim3(kThreads), lds, s, a); break;
        case 96: hipLaunchKernelGGL((decode_window_kernel<DT, 96>), grid, dim3(kThreads), lds, s, a); break;
        case 128: hipLaunchKernelGGL((decode_window_kernel<DT, 128>), grid, dim3(kThreads), lds, s, a); break;
        case 160: hipLaunchKernelGGL((decode_window_kernel<DT, 160>), grid, dim3(kThreads), lds, s, a); break;
        case 192: hipLaunchKernelGGL((decode_window_kernel<DT, 192>), grid, dim3(kThreads), lds, s, a); break;
        case 224: hipLaunchKernelGGL((decode_window_kernel<DT, 224>), grid, dim3(kThreads), lds, s, a); break;
        default: hipLaunchKernelGGL((decode_window_kernel<DT, 256>), grid, dim3(kThreads), lds, s, a); break;
    }
}

hipError_t launch_decode_window(const DecodeArgs& a, hipStream_t s) {
    const int RA = a.q_heads / a.kv_heads, R = std::min(RA, kWinHeads);
    dim3 grid(a.win_splits, a.kv_heads * ((RA + kWinHeads - 1) / kWinHeads), a.num_seqs * a.n_layers);
    const int TP = kThreads / a.head_dim;
    const size_t lds = sizeof(float) * ((size_t)R * a.head_dim + (size_t)R * kWinTokens + 2 * R +
                                        (TP > 1 ? (size_t)TP * R * a.head_dim : 0)) +
                       sizeof(int) * 2 * kWinTokens + 8 + sizeof(double) * (a.head_dim / 2);
    switch (a.in_dtype) {
        case 0: window_d<0>(a, grid, lds, s); break;
        case 1: window_d<1>(a, grid, lds, s); break;
        default: window_d<2>(a, grid, lds, s); break;
    }
    return hipGetLastError();
}

hipError_t launch_dequant(const DequantArgs& a, hipStream_t s) {
    const int units = a.len * (a.head_dim >> 5);
    if (units == 0) return hipSuccess;
    dim3 grid((units + kThreads - 1) / kThreads, a.kv_heads);
    switch (a.in_dtype) {
        case 0: hipLaunchKernelGGL(dequant_kernel<0>, grid, dim3(kThreads), 0, s, a); break;
        case 1: hipLaunchKernelGGL(dequant_kernel<1>, grid, dim3(kThreads), 0, s, a); break;
        default: hipLaunchKernelGGL(dequant_kernel<2>, grid, dim3(kThreads), 0, s, a); break;
    }
    return hipGetLastError();
}


// ---------------------------------------------------------------- page lists
namespace {
__global__ __launch_bounds__(kThreads) void page_update_kernel(uint32_t* pages, PageUpdates u) {
    const int i = blockIdx.x * kThreads + threadIdx.x;
    if (i < u.count) pages[u.index[i]] = u.value[i];
}
}  // namespace

hipError_t launch_page_updates(uint32_t* pages, const PageUpdates& u, hipStream_t s) {
    if (u.count <= 0) return hipSuccess;
    hipLaunchKernelGGL(page_update_kernel, dim3((u.count + kThreads - 1) / kThreads), dim3(kThreads), 0, s, pages, u);
    return hipGetLastError();
}

// ---------------------------------------------------------------- read probe
// A plain streaming read (the measured HBM ceiling the decode kernels are
// compared with): grid-stride 16-byte non-temporal loads, four in flight per
// lane, folded into one word that is stored only if it equals a constant no
// input is expected to produce (the loads cannot be elided).
namespace {
typedef unsigned int probe_u32x4 __attribute__((ext_vector_type(4)));
__global__ __launch_bounds__(256) void read_probe_kernel(const probe_u32x4* __restrict__ p, size_t n, uint32_t* sink) {
    const size_t stride = (size_t)gridDim.x * 256;
    size_t i = (size_t)blockIdx.x * 256 + threadIdx.x;
    uint32_t acc = 0;
    for (; i + 3 * stride < n; i += 4 * stride) {
        probe_u32x4 v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = __builtin_nontemporal_load(p + i + u * stride);
#pragma unroll
        for (int u = 0; u < 4; ++u) acc ^= v[u].x ^ v[u].y ^ v[u].z ^ v[u].w;
    }
    for (; i < n; i += stride) {
        const probe_u32x4 v = __builtin_nontemporal_load(p + i);
        acc ^= v.x ^ v.y ^ v.z ^ v.w;
    }
    if (acc == 0x9e3779b9u) *sink = acc;
}
}  // namespace

hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s) {
    const size_t n = bytes / 16;
    const int grid = 8192;  // 32 waves per CU: the fastest launch shape measured for this loop
    hipLaunchKernelGGL(read_probe_kernel, dim3(grid), dim3(256), 0, s, (const probe_u32x4*)buf, n, sink);
    return hipGetLastError();
}

}  // namespace kvq
