// Device helpers shared by the HIP kernels of libkvq (internal).
#pragma once

#include <hip/hip_runtime.h>

#include <utility>

#include "kvq_internal.h"

namespace kvq {
namespace dev {

// f(integral_constant<int, I>) for I = 0..N-1, unrolled at compile time.
template <typename F, int... I>
__device__ __forceinline__ void static_for_impl(F& f, std::integer_sequence<int, I...>) {
    (f(std::integral_constant<int, I>{}), ...);
}
template <int N, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    static_for_impl(f, std::make_integer_sequence<int, N>{});
}

// Streaming loads of the quantized cache, which a decode step reads exactly
// once: the non-temporal hint keeps them from displacing reused lines and
// measured ~9% more read bandwidth than plain loads on a 1 GiB stream.
typedef unsigned int u32x2_t __attribute__((ext_vector_type(2)));
typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t ld_stream(const uint32_t* p) {
    return __builtin_nontemporal_load(p);
}
__device__ __forceinline__ uint2 ld_stream2(const uint32_t* p) {
    const u32x2_t v = __builtin_nontemporal_load((const u32x2_t*)p);
    return make_uint2(v.x, v.y);
}
__device__ __forceinline__ uint4 ld_stream4(const uint32_t* p) {
    const u32x4_t v = __builtin_nontemporal_load((const u32x4_t*)p);
    return make_uint4(v.x, v.y, v.z, v.w);
}

// The arguments of the layer that workgroup index z of a multi-layer launch
// serves (per_layer indices per layer); z becomes the index within the layer.
__device__ __forceinline__ DecodeArgs layer_args(const DecodeArgs& a0, int& z, int per_layer) {
    if (a0.n_layers <= 1) return a0;
    const int lz = z / per_layer;
    z -= lz * per_layer;
    DecodeArgs a = a0;
    const size_t rows = (size_t)lz * a.num_seqs * a.q_heads;  // query rows of the layers before
    a.table += (size_t)lz * a.num_seqs;
    a.len = a.len_base + ((size_t)((a.len_parity >> lz) & 1u) * a.layers_total + a.layer0 + lz) * a.num_seqs;
    a.q = (const uint8_t*)a.q + rows * a.head_dim * (a.in_dtype == 0 ? 4 : 2);
    a.out += rows * a.head_dim;
    a.ws_ml += rows * a.max_chunks * 2;
    a.ws_o += rows * a.max_chunks * a.head_dim;
    return a;
}

// The same for one tensor of a multi-layer append (grid z = layer * num_seqs + seq).
__device__ __forceinline__ TensorArgs layer_args(const TensorArgs& a0, int& z, int per_layer) {
    if (a0.n_layers <= 1) return a0;
    const int lz = z / per_layer;
    z -= lz * per_layer;
    TensorArgs a = a0;
    const size_t p = (a.len_parity >> lz) & 1u;
    a.table += (size_t)lz * a.num_seqs;
    a.len_in = a.len_base + (p * a.layers_total + a.layer0 + lz) * a.num_seqs;
    if (a0.len_out) a.len_out = a.len_base + ((1 - p) * a.layers_total + a.layer0 + lz) * a.num_seqs;
    a.src = (const uint8_t*)a.src + lz * a.src_layer_bytes;
    return a;
}

// Full-precision window and sinks: the tokens [tb, te) a decode kernel reads
// quantized, the whole key blocks inside [sinks, len - window); everything else
// below len is read in full precision. Without a window, [0, len).
__device__ __forceinline__ void quant_range(const DecodeArgs& a, int len, int& tb, int& te) {
    if (!a.win_mode) {
        tb = 0;
        te = len;
        return;
    }
    const int r = len - a.window;
    const int q = r > 0 ? r / a.tblock * a.tblock : 0;
    tb = a.sinks;
    te = q > a.sinks ? q : a.sinks;
}

// Quantized splits of [tb, te) (window mode): split_floor 1 -> the single-query
// kernel's max(1, n / chunk), else ceil(n / chunk); 0 when the range is empty.
__device__ __forceinline__ int quant_splits(const DecodeArgs& a, int tb, int te) {
    const int n = te - tb;
    if (n <= 0) return 0;
    return a.split_floor ? (n / a.chunk > 1 ? n / a.chunk : 1) : (n + a.chunk - 1) / a.chunk;
}

// Full-precision tokens of a sequence of length len (window mode): the sinks
// [0, min(sinks, len)) then the recent tokens [max(te, sinks), len); fp_token(i)
// is the i-th of them and window_row(t) its row in the head's window area.
__device__ __forceinline__ int fp_count(const DecodeArgs& a, int len, int te) {
    const int ns = len < a.sinks ? len : a.sinks;
    const int rs = te > ns ? te : ns;
    return ns + (len > rs ? len - rs : 0);
}
__device__ __forceinline__ int fp_token(const DecodeArgs& a, int len, int te, int i) {
    const int ns = len < a.sinks ? len : a.sinks;
    const int rs = te > ns ? te : ns;
    return i < ns ? i : rs + (i - ns);
}
// ring: the sequence's ring offset (tokens evicted before the window, mod win_rows)
__device__ __forceinline__ int window_row(int t, int sinks, int win_rows, int ring) {
    return t < sinks ? t : sinks + (t + ring) % win_rows;
}

// 2^x (v_exp_f32) for results that inline asm reads. On gfx940-class parts a
// VALU instruction that reads the result of a transcendental one (exp, log,
// rcp, ...) in the very next slot gets the old register contents; the
// compiler inserts the wait state for its own instructions but does not look
// inside asm blocks, so an asm consumer scheduled right after the exp read a
// stale value. The wait state travels with the exp here, whatever follows it.
__device__ __forceinline__ float exp2_for_asm(float x) {
    float d;
    asm("v_exp_f32 %0, %1\n\ts_nop 0" : "=v"(d) : "v"(x));
    return d;
}

// Token t of a table entry: the byte offset of its page in the codes pool (the
// metadata pool too with paged storage) and its row inside the page. Both
// storages take the same path: a contiguous entry has one page at offset 0
// (page_bytes 0) whose rows are the tokens themselves.
struct PageRow {
    uint64_t base;
    int row;
};
__device__ __forceinline__ PageRow page_row(const uint32_t* pages, const SeqEntry& e, int t) {
    return {(uint64_t)pages[e.page_list + (t >> e.page_shift)] * e.page_bytes, t & ((1 << e.page_shift) - 1)};
}

__device__ __forceinline__ float f16_to_f32(uint32_t bits16) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)(bits16 & 0xffffu));
}
__device__ __forceinline__ uint32_t f32_to_f16_bits(float f) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)f);
}
__device__ __forceinline__ float bf16_to_f32(uint32_t bits16) {
    return __uint_as_float((bits16 & 0xffffu) << 16);
}

// Input dtype tags: 0 = f32, 1 = f16, 2 = bf16.
template <int DT> struct In;
template <> struct In<0> { static constexpr int bytes = 4; };
template <> struct In<1> { static constexpr int bytes = 2; };
template <> struct In<2> { static constexpr int bytes = 2; };

template <int DT>
__device__ __forceinline__ float load_in(const void* p, size_t i) {
    if constexpr (DT == 0) {
        return ((const float*)p)[i];
    } else if constexpr (DT == 1) {
        return f16_to_f32(((const uint16_t*)p)[i]);
    } else {
        return bf16_to_f32(((const uint16_t*)p)[i]);
    }
}

template <int DT>
__device__ __forceinline__ float half_to_f32(uint32_t h) {
    if constexpr (DT == 1) return f16_to_f32(h);
    else return bf16_to_f32(h);
}

// Keys cached before the rotary embedding ([U] "Embebedos Rotatorios
// Complicam as Chaves"): cos and sin of the angle t * theta, reduced modulo
// 2 pi in float64 (t * theta reaches 1e5-1e8 radians at long context, where a
// float32 product would be off by 1e-2 rad), then evaluated in float32.
__device__ __forceinline__ void rope_cs(int t, double theta, float& c, float& s) {
    const double ang = (double)t * theta;
    const double r = ang - 6.283185307179586 * rint(ang * 0.15915494309189535);
    sincosf((float)r, &s, &c);
}

// 16 consecutive input elements starting at element `off`.
template <int DT>
__device__ __forceinline__ void load16(const void* base, size_t off, float (&x)[16]) {
#pragma unroll
    for (int j = 0; j < 16; ++j) x[j] = load_in<DT>(base, off + j);
}

// 32 consecutive input elements starting at element `off` (16-byte aligned).
template <int DT>
__device__ __forceinline__ void load32(const void* base, size_t off, float (&x)[32]) {
    if constexpr (DT == 0) {
        const uint4* p = (const uint4*)((const float*)base + off);
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint4 v = p[i];
            x[4 * i + 0] = __uint_as_float(v.x);
            x[4 * i + 1] = __uint_as_float(v.y);
            x[4 * i + 2] = __uint_as_float(v.z);
            x[4 * i + 3] = __uint_as_float(v.w);
        }
    } else {
        const uint4* p = (const uint4*)((const uint16_t*)base + off);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint4 v = p[i];
            const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
            for (int k = 0; k < 4; ++k) {
                x[8 * i + 2 * k + 0] = half_to_f32<DT>(w[k]);
                x[8 * i + 2 * k + 1] = half_to_f32<DT>(w[k] >> 16);
            }
        }
    }
}

// The reciprocal quant_code takes for a stored step s, once per group: 0 for
// a zero step, whose codes are all 0 (every product is then 0).
__device__ __forceinline__ float quant_rcp(float s) { return s == 0.0f ? 0.0f : __builtin_amdgcn_rcpf(s); }

// Code of one value against the stored grid (step s, zero z), L = 2^B - 1:
// clamp(rint((x - z) / s), 0, L) with the correctly rounded fp32 quotient and
// ties to even, 0 where s = 0. The quotient is taken as (x - z) * r, r =
// quant_rcp(s), within 2^-21 of it relative (reciprocal and product roundings,
// the quotient's own), clamped, and rounded to an integer by the fp32 adder
// (t + 2^23 keeps the integer part, ties to even). For t <= 255 the two can
// round apart only when the product lies within 2^-13 of a half-integer;
// there the quotient is divided out (about 2 elements in 10^4; never for s =
// 0, where t = 0).
__device__ __forceinline__ uint32_t quant_code(float x, float r, float s, float z, float L) {
    const float a = x - z;
    const float t = __builtin_amdgcn_fmed3f(a * r, 0.0f, L);
    const float m = t + 8388608.0f;
    if (fabsf(fabsf(t - (m - 8388608.0f)) - 0.5f) < 0x1p-13f)
        return (uint32_t)__builtin_amdgcn_fmed3f(rintf(a / s), 0.0f, L);
    return __float_as_uint(m) & 0xffu;
}

// Pack 32 codes into the B words of one unit: code j at stream bits [jB, jB+B).
template <int B>
__device__ __forceinline__ void pack32(const uint32_t (&c)[32], uint32_t (&w)[B]) {
#pragma unroll
    for (int k = 0; k < B; ++k) w[k] = 0u;
#pragma unroll
    for (int j = 0; j < 32; ++j) {
        const int pos = j * B, wi = pos >> 5, sh = pos & 31;
        w[wi] |= c[j] << sh;
        if (sh + B > 32) w[wi + 1] |= c[j] >> (32 - sh);
    }
}

template <int B>
__device__ __forceinline__ uint32_t code_at(const uint32_t (&w)[B], int j) {
    const int pos = j * B, wi = pos >> 5, sh = pos & 31;
    uint32_t v = w[wi] >> sh;
    if (sh + B > 32) v |= w[wi + 1] << (32 - sh);
    return v & ((1u << B) - 1u);
}

template <int B>
__device__ __forceinline__ void load_unit(const uint32_t* p, uint32_t (&w)[B]) {
#pragma unroll
    for (int k = 0; k < B; ++k) w[k] = p[k];
}

template <int B>
__device__ __forceinline__ void store_codes(const uint32_t (&c)[32], uint32_t* dst) {
    uint32_t w[B];
    pack32<B>(c, w);
#pragma unroll
    for (int k = 0; k < B; ++k) dst[k] = w[k];
}

__device__ __forceinline__ void store_codes_rt(int B, const uint32_t (&c)[32], uint32_t* dst) {
    switch (B) {
        case 2: store_codes<2>(c, dst); break;
        case 3: store_codes<3>(c, dst); break;
        case 4: store_codes<4>(c, dst); break;
        case 6: store_codes<6>(c, dst); break;
        default: store_codes<8>(c, dst); break;
    }
}

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v += __shfl_xor(v, off);
    return v;
}
__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int off = 32; off > 0; off >>= 1) v = fmaxf(v, __shfl_xor(v, off));
    return v;
}

// Workgroup-wide reductions over 256 threads (4 waves); `scratch` holds 4 floats.
__device__ __forceinline__ float block_sum(float v, float* scratch) {
    v = wave_sum(v);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[wave] = v;
    __syncthreads();
    return (scratch[0] + scratch[1]) + (scratch[2] + scratch[3]);
}
__device__ __forceinline__ float block_max(float v, float* scratch) {
    v = wave_max(v);
    const int wave = threadIdx.x >> 6;
    __syncthreads();
    if ((threadIdx.x & 63) == 0) scratch[wave] = v;
    __syncthreads();
    return fmaxf(fmaxf(scratch[0], scratch[1]), fmaxf(scratch[2], scratch[3]));
}

}  // namespace dev
}  // namespace kvq
