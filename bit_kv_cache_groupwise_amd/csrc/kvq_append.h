// Device code of the quantize-append shared by the append kernel and the
// fused decode step (internal): the token-axis rows and the residual-row copy.
#pragma once

#include "kvq_device.h"
#include "kvq_internal.h"

namespace kvq {
namespace dev {

// ---------------------------------------------------------------------------
// Quantize, token axis: one group = G consecutive channels of one token
// ([U] "Valores: Onde a Intuicao Quebra"; [U] "O Imposto dos Sistemas ...":
// such groups are complete when their token arrives). One thread per
// 32-channel unit; a group spans G/32 adjacent lanes and its min/max is a
// butterfly over those lanes. Workgroup `item` takes rows item*rows_per_block..
// ---------------------------------------------------------------------------
// Row r (< n) of the new rows of (seq, head), 32-channel unit u: one thread
// per unit; the lanes of a row are consecutive and leave or stay together.
template <int DT>
__device__ __forceinline__ void token_axis_row(const TensorArgs& a, int r, int u, int head, int seq, int len0) {
    const int D = a.head_dim;
    const int row_start = a.row_start ? a.row_start[seq] : seq * a.n_uniform;
    const SeqEntry& e = a.table[seq];
    const int T = a.tensor, B = e.bits[T], G = a.group, UG = G >> 5;
    const int t = len0 + r;

    float x[32];
    load32<DT>(a.src, ((size_t)(row_start + r) * a.kv_heads + head) * D + 32 * u, x);
    float mn = x[0], mx = x[0];
#pragma unroll
    for (int j = 1; j < 32; ++j) {
        mn = fminf(mn, x[j]);
        mx = fmaxf(mx, x[j]);
    }
    for (int off = 1; off < UG; off <<= 1) {
        mn = fminf(mn, __shfl_xor(mn, off));
        mx = fmaxf(mx, __shfl_xor(mx, off));
    }
    const float L = (float)((1 << B) - 1);
    const float s32 = (mx - mn) / L;
    const uint32_t sb = f32_to_f16_bits(s32), zb = f32_to_f16_bits(mn);
    const float s = f16_to_f32(sb), z = f16_to_f32(zb);
    const PageRow pr = page_row(a.pages, e, t);
    uint32_t* meta = (uint32_t*)(a.meta + pr.base + e.meta[T] + (size_t)head * e.meta_hs[T]);
    if ((u & (UG - 1)) == 0) meta[(size_t)pr.row * (D / G) + u / UG] = sb | (zb << 16);
    const float rs = quant_rcp(s);
    uint32_t c[32];
#pragma unroll
    for (int j = 0; j < 32; ++j) c[j] = quant_code(x[j], rs, s, z, L);
    uint32_t* dst =
        (uint32_t*)(a.codes + pr.base + e.codes[T] + (size_t)head * e.codes_hs[T] + (size_t)pr.row * (D * B / 8)) +
        u * B;
    store_codes_rt(B, c, dst);
}

template <int DT>
__device__ __forceinline__ void token_axis_part(const TensorArgs& a, int item, int head, int seq) {
    const int UPR = a.head_dim >> 5;
    const int len0 = a.len_in[seq];
    const int n = a.n_new ? a.n_new[seq] : a.n_uniform;
    if (a.len_out && item == 0 && head == 0 && threadIdx.x == 0) a.len_out[seq] = len0 + n;
    const int r = item * a.rows_per_block + (int)threadIdx.x / UPR;
    if (r < n) token_axis_row<DT>(a, r, (int)threadIdx.x % UPR, head, seq, len0);
}

// Copy new rows t in [start, len0 + n) of (seq, head) into the residual, row t % G
// (the rows of the channel-axis block still incomplete after the append).
template <int DT>
__device__ __forceinline__ void residual_rows(const TensorArgs& a, int head, int seq, int start, int len0, int len1,
                                              int nthreads) {
    constexpr int IB = In<DT>::bytes;
    const int D = a.head_dim;
    const int row_start = a.row_start ? a.row_start[seq] : seq * a.n_uniform;
    const SeqEntry& e = a.table[seq];
    uint8_t* rw = a.resid + e.resid[a.tensor] + (size_t)head * e.resid_hs[a.tensor];
    const int count = (len1 - start) * D;
    for (int idx = threadIdx.x; idx < count; idx += nthreads) {
        const int i = idx / D, ch = idx % D;
        const int t = start + i;
        const size_t so = ((size_t)(row_start + t - len0) * a.kv_heads + head) * D + ch;
        const size_t dof = (size_t)(t % a.group) * D + ch;
        if constexpr (IB == 4) ((uint32_t*)rw)[dof] = ((const uint32_t*)a.src)[so];
        else ((uint16_t*)rw)[dof] = ((const uint16_t*)a.src)[so];
    }
}

// Copy the new rows of an append that the full-precision window keeps into the
// window area of (seq, head): sink tokens t < sinks, and the later tokens
// t >= len1 - win_rows (no two of them share a row). One element per thread,
// keys and values; workgroup `item` of `nitems` takes every nitems-th block of
// nthreads elements.
template <int DT>
__device__ __forceinline__ void window_rows(const TensorArgs& k, const TensorArgs& v, int seq, int head, int item,
                                            int nitems, int nthreads) {
    const int D = k.head_dim;
    const int len0 = k.len_in[seq];
    const int n = k.n_new ? k.n_new[seq] : k.n_uniform;
    const int row_start = k.row_start ? k.row_start[seq] : seq * k.n_uniform;
    const int len1 = len0 + n;
    // kept rows: sinks [len0, min(len1, sinks)), then [max(len0, sinks, len1 - win_rows), len1)
    const int n1 = max(0, min(len1, k.sinks) - len0);
    const int s2 = max(max(len0, k.sinks), len1 - k.win_rows);
    const int n2 = max(0, len1 - s2);
    constexpr int IB = In<DT>::bytes;
    const SeqEntry& e = k.table[seq];
    for (int idx = item * nthreads + (int)threadIdx.x; idx < (n1 + n2) * D; idx += nitems * nthreads) {
        const int j = idx / D, ch = idx % D;
        const int t = j < n1 ? len0 + j : s2 + (j - n1), i = t - len0;
        const size_t so = ((size_t)(row_start + i) * k.kv_heads + head) * D + ch;
        const size_t dof = (size_t)window_row(t, k.sinks, k.win_rows, e.ring) * D + ch;
#pragma unroll
        for (int T = 0; T < 2; ++T) {
            const TensorArgs& x = T == 0 ? k : v;
            uint8_t* w = x.resid + e.resid[T] + (size_t)head * e.resid_hs[T] + x.win_off;
            if constexpr (IB == 4) ((uint32_t*)w)[dof] = ((const uint32_t*)x.src)[so];
            else ((uint16_t*)w)[dof] = ((const uint16_t*)x.src)[so];
        }
    }
}

}  // namespace dev
}  // namespace kvq
