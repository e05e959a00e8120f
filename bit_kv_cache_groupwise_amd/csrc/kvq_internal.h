// Internal declarations shared by the host side of libkvq (kvq_api.cpp) and
// its HIP kernels (kvq_kernels.hip). Not part of the public ABI.
#pragma once

#include <stddef.h>
#include <stdint.h>

#include <hip/hip_runtime_api.h>

namespace kvq {

constexpr int kMaxHeadDim = 256;
constexpr int kMaxQueryGroup = 16;  // q_heads / kv_heads handled by one decode workgroup
constexpr int kThreads = 256;       // threads per workgroup of every kernel
constexpr uint64_t kAlign = 256;    // alignment of every head region and pool

// One (layer, seq) entry of the device table. Byte offsets into the codes,
// metadata and residual pools of head 0 of each tensor, and per-head strides.
// Codes and metadata are addressed through pages: token t lies in physical
// page pages[page_list + (t >> page_shift)], at byte pool offset page *
// page_bytes, row t & (2^page_shift - 1) of the page; codes[] and meta[] are
// offsets inside the page. Contiguous storage is the case of one page per
// (layer, seq): page_shift 30, page_bytes 0 and a page list holding 0, so that
// the offsets are pool offsets and the row is t.
constexpr int kContiguousShift = 30;
struct SeqEntry {
    uint64_t codes[2];        // [K, V]
    uint64_t meta[2];
    uint64_t resid[2];
    uint64_t codes_hs[2];
    uint64_t meta_hs[2];
    uint64_t resid_hs[2];
    uint64_t page_bytes;      // stride of physical pages (0: contiguous)
    int32_t bits[2];
    int32_t cap;
    int32_t page_shift;       // log2 tokens per page
    uint32_t page_list;       // first entry of this (layer, seq)'s page list
    int32_t ring;             // window mode: token t >= sinks lives in ring row (t + ring) % win_rows
};
static_assert(sizeof(SeqEntry) == 128, "SeqEntry layout");
constexpr uint32_t kNoPage = 0xffffffffu;

// Table buffer layout (bytes from d_table):
//   [0, entries_bytes)                 SeqEntry[layers][num_seqs]
//   [len_off, +2*layers*num_seqs*4)    int32 lengths[2][layers][num_seqs] (double buffered)
//   [args_off, +2*num_seqs*4)          int32 call args: n_new[num_seqs], row_start[num_seqs]
//   [ctr_off, +num_seqs*kv_heads*4)    int32 split counters of the decode merge (zero between calls)
//   [pairs_off, +num_seqs*4)           int32 sequence indices grouped by (bits_k, bits_v) pair
//   [pt_off, +page_entries*4)          uint32 page lists (contiguous storage: one entry, 0)
struct TableLayout {
    uint64_t entries_bytes, len_off, args_off, ctr_off, pairs_off, pt_off, rope_off, total;
};

// Per-launch description of one tensor (K = 0 or V = 1) of one layer.
struct TensorArgs {
    const void* src;            // new rows [sum n][Hkv][D], input dtype
    uint8_t* codes;             // codes pool
    uint8_t* meta;              // metadata pool
    uint8_t* resid;             // residual pool
    const SeqEntry* table;      // entries of this layer: table[seq]
    const int32_t* len_in;      // lengths of this layer before the call [num_seqs]
    int32_t* len_out;           // lengths after the call (other buffer), or nullptr
    const int32_t* n_new;       // device [num_seqs] or nullptr when uniform
    const int32_t* row_start;   // device [num_seqs] or nullptr when uniform
    int32_t n_uniform;
    int32_t tensor;             // 0 = K, 1 = V
    int32_t num_seqs, kv_heads, head_dim, group, in_dtype;
    int32_t rows_per_block;     // token axis: rows per workgroup
    int32_t axis;               // KVQ_AXIS_CHANNEL (0) or KVQ_AXIS_TOKEN (1)
    // Several consecutive layers in one launch (n_layers > 1): the grid's z
    // runs over n_layers ranges of num_seqs, one per layer (layer_args()).
    int32_t n_layers;           // 1 for a single-layer call
    int32_t layers_total, layer0;
    uint64_t len_parity;        // bit i: current length buffer of layer layer0 + i
    int32_t* len_base;          // both length buffers, [2][layers_total][num_seqs]
    uint64_t src_layer_bytes;   // bytes of new rows per layer in src
    // Full-precision window and sinks (win_mode != 0): new rows are also copied
    // into the window area of the head's residual region (window_store_kernel).
    int32_t win_mode, sinks, win_rows;  // win_rows = window + block (the recent ring)
    uint32_t win_off;           // byte offset of the window area inside a head's residual region
    const uint32_t* pages;      // page lists (SeqEntry::page_list indexes them)
};

struct DecodeArgs {
    const void* q;              // [S][Hq][D], input dtype
    float* out;                 // [S][Hq][D]
    float* ws_ml;               // [S][Hq][max_chunks][2]
    float* ws_o;                // [S][Hq][max_chunks][D]
    const uint8_t* codes;
    const uint8_t* meta;
    const uint8_t* resid;
    const SeqEntry* table;      // entries of this layer
    const int32_t* len;         // lengths of this layer [num_seqs]
    float qscale;               // softmax scale * log2(e)
    int32_t num_seqs, kv_heads, q_heads, head_dim;
    int32_t group_k, group_v, axis_k, axis_v, in_dtype;
    int32_t chunk;              // tokens per split (multiple of group_k when axis_k is channel)
    int32_t max_chunks;         // chunks per (seq, head) the workspace is laid out for
    const int32_t* seq_list;    // blockIdx.z -> sequence (single-query kernel), or nullptr
    int32_t* counters;          // [num_seqs][kv_heads] split counters (reserved)
    int32_t split_floor;        // splits per seq: 0 -> ceil(len/chunk), 1 -> max(1, len/chunk)
    int32_t log2_group_k, log2_group_v;
    int32_t waves_per_group;    // single-query kernel: waves per workgroup (4)
    // Several consecutive layers in one launch (n_layers > 1): the grid's
    // sequence index (z of the decode grids, y of the merge grid) runs over
    // n_layers equal ranges, one per layer; layer_args() maps a workgroup to
    // its layer's table, lengths, q, out and workspace slices.
    int32_t n_layers;           // 1 for a single-layer call
    int32_t layers_total;       // layers of the cache
    int32_t layer0;             // first layer of the launch
    uint64_t len_parity;        // bit i: current length buffer of layer layer0 + i
    const int32_t* len_base;    // both length buffers, [2][layers_total][num_seqs]
    // Fused decode step (append_fused != 0; single-query kernel, one layer):
    // the last split of each (seq, kv head) first appends that sequence's new
    // rows (values quantized on the token axis, keys copied into the residual;
    // no key block completes in the step), then attends with the post-append
    // length. `len` then holds the lengths before the append.
    int32_t append_fused;
    TensorArgs app_k, app_v;
    // Full-precision window and sinks (win_mode != 0): the quantized kernels
    // read tokens [sinks, Q) only (quant_range) and always write split
    // partials; decode_window_kernel writes the full-precision rows' partials
    // after them (slots nq .. nq + nfs - 1) and merge_kernel merges both.
    int32_t win_mode, window, sinks, tblock, win_rows;  // tblock: key block in tokens
    uint32_t win_off[2];        // byte offset of the window area inside a head's residual region [K, V]
    float ws_scale;             // factor the quantized kernel's partial l and o carry (2^24: single query)
    int32_t win_splits;         // grid x of decode_window_kernel (full-precision splits at most)
    // Keys cached before the rotary embedding (rope_base > 0): the
    // reconstructed key of token t is rotated to position t.
    double rope_base;
    // Rotary tables of the cache (rope_base > 0): theta_i = base^(-2i/D) for
    // the D/2 pairs (i, i + D/2), and (cos, sin)(u theta_i) for the in-tile
    // offsets u = 0..kRopeRows-1, row-major [u][i] as float pairs.
    const double* rope_theta;
    const float* rope_tab;
    const uint32_t* pages;      // page lists (SeqEntry::page_list indexes them)
};

struct DequantArgs {
    float* out;                 // [Hkv][len][D]
    const uint8_t* codes;
    const uint8_t* meta;
    const uint8_t* resid;
    SeqEntry entry;
    int32_t tensor, len, kv_heads, head_dim, group, axis, in_dtype;
    int32_t win_mode, window, sinks, tblock, win_rows;  // as in DecodeArgs
    uint32_t win_off;
    const uint32_t* pages;      // page lists (SeqEntry::page_list indexes them)
};

// Work list of the query-group kernel when one launch covers every bit pair of
// a call: entry k = one (layer, seq) with start[k] its first workgroup; the
// entries are ordered by bit pair and start[count] is the total. Passed by
// value in the kernel arguments.
// Rows of the rotary (cos, sin) table: in-tile offsets 0..31 and the step 32
// between the two 32-token halves of a 64-token tile.
constexpr int kRopeRows = 33;

constexpr int kGqaListMax = 256;
struct GqaList {
    int32_t count;
    int32_t start[kGqaListMax + 1];
    uint16_t seq[kGqaListMax];
    uint8_t layer[kGqaListMax];  // offset from the call's first layer
};

constexpr int kWinTokens = 64;  // full-precision tokens per decode_window_kernel workgroup
constexpr int kWinHeads = 4;    // query heads per decode_window_kernel workgroup

// Channel-axis quantization by one wave per block (four blocks per workgroup),
// with the block's inputs held in registers (one channel pair per lane): blocks
// of 32 tokens, head_dim <= 128. Other blocks take one workgroup per block, two
// passes over the inputs.
constexpr int kQuantBlocksPerGroup = 4;
// Channel-axis blocks quantized by one wave each (the block's G x D tile read
// once into registers, G * D / 64 input values per lane): 32-token blocks at
// head_dim <= 128 for every input type; for 2-byte inputs also 32-token blocks
// at head_dim <= 256 and 64-token blocks at head_dim <= 64.
constexpr bool quant_wave_path(int group, int head_dim, int in_dtype) {
    return (group == 32 && head_dim <= 128) ||
           (in_dtype != 0 && ((group == 32 && head_dim <= 256) || (group == 64 && head_dim <= 64)));
}
// Resident workgroups per compute unit of the query-group kernel (4 waves, one
// per SIMD each): the waves-per-SIMD bound each of its objects is built with
// (KVQ_GQA_OCCUPANCY: 3 below head_dim 256, 2 at 256; rotary keys 2 and 1).
// The split choice runs its workgroups in rounds of this count.
constexpr int gqa_resident_per_cu(int head_dim, bool rope) {
    return rope ? (head_dim >= 256 ? 1 : 2) : (head_dim >= 256 ? 2 : 3);
}

// the wave path's larger tile (two channel pairs per lane)
constexpr bool quant_wave_wide(int group, int head_dim) { return group == 32 && head_dim > 128; }

// Keys and values of one append in one launch: gx_k workgroups per (head, seq)
// for the keys, then gx_v for the values, then (window mode) the copy of the
// rows the full-precision window keeps (max_new: most tokens a sequence appends).
hipError_t launch_quant_append(const TensorArgs& k, const TensorArgs& v, int gx_k, int gx_v, int max_new,
                               hipStream_t s);
hipError_t launch_decode(const DecodeArgs& a, hipStream_t s);
hipError_t launch_merge(const DecodeArgs& a, hipStream_t s);
hipError_t launch_decode_mha_d64(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
hipError_t launch_decode_mha_d128(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
hipError_t launch_decode_mha_d256(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
hipError_t launch_decode_gqa_d64(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
hipError_t launch_decode_gqa_d128(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
hipError_t launch_decode_gqa_d256(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
hipError_t launch_decode_gqa_list_d64(const DecodeArgs& a, const GqaList& list, int items, hipStream_t s);
hipError_t launch_decode_gqa_list_d128(const DecodeArgs& a, const GqaList& list, int items, hipStream_t s);
hipError_t launch_decode_gqa_list_d256(const DecodeArgs& a, const GqaList& list, int items, hipStream_t s);
inline hipError_t launch_decode_gqa_list(const DecodeArgs& a, const GqaList& list, int items, hipStream_t s) {
    return a.head_dim == 64    ? launch_decode_gqa_list_d64(a, list, items, s)
           : a.head_dim == 128 ? launch_decode_gqa_list_d128(a, list, items, s)
                               : launch_decode_gqa_list_d256(a, list, items, s);
}
inline hipError_t launch_decode_gqa(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s) {
    return a.head_dim == 64    ? launch_decode_gqa_d64(a, bits_k, bits_v, nseqs, s)
           : a.head_dim == 128 ? launch_decode_gqa_d128(a, bits_k, bits_v, nseqs, s)
                               : launch_decode_gqa_d256(a, bits_k, bits_v, nseqs, s);
}
// Keys cached before the rotary embedding on the query-group kernel (head_dim 128 and 256).
hipError_t launch_decode_gqa_rope_list_d128(const DecodeArgs& a, const GqaList& list, int items, hipStream_t s);
hipError_t launch_decode_gqa_rope_list_d256(const DecodeArgs& a, const GqaList& list, int items, hipStream_t s);
hipError_t launch_decode_gqa_rope_d128(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
hipError_t launch_decode_gqa_rope_d256(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
inline bool gqa_rope_supported(int head_dim) { return head_dim == 128 || head_dim == 256; }
inline bool mha_supported(int head_dim) { return head_dim == 64 || head_dim == 128 || head_dim == 256; }
bool mha_fused_ok_d64(int bits_k, int bits_v);
bool mha_fused_ok_d128(int bits_k, int bits_v);
bool mha_fused_ok_d256(int bits_k, int bits_v);
// Whether the fused decode step keeps the single-query kernel's occupancy for this bit pair.
inline bool mha_fused_ok(int head_dim, int bits_k, int bits_v) {
    return head_dim == 64    ? mha_fused_ok_d64(bits_k, bits_v)
           : head_dim == 128 ? mha_fused_ok_d128(bits_k, bits_v)
                             : mha_fused_ok_d256(bits_k, bits_v);
}
inline hipError_t launch_decode_mha(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s) {
    return a.head_dim == 64    ? launch_decode_mha_d64(a, bits_k, bits_v, nseqs, s)
           : a.head_dim == 128 ? launch_decode_mha_d128(a, bits_k, bits_v, nseqs, s)
                               : launch_decode_mha_d256(a, bits_k, bits_v, nseqs, s);
}
// Keys cached before the rotary embedding on the single-query kernel (its
// rotary instantiations, one object per head_dim).
hipError_t launch_decode_mha_rope_d64(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
hipError_t launch_decode_mha_rope_d128(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
hipError_t launch_decode_mha_rope_d256(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s);
bool mha_rope_fused_ok_d64(int bits_k, int bits_v);
bool mha_rope_fused_ok_d128(int bits_k, int bits_v);
bool mha_rope_fused_ok_d256(int bits_k, int bits_v);
inline bool mha_rope_fused_ok(int head_dim, int bits_k, int bits_v) {
    return head_dim == 64    ? mha_rope_fused_ok_d64(bits_k, bits_v)
           : head_dim == 128 ? mha_rope_fused_ok_d128(bits_k, bits_v)
                             : mha_rope_fused_ok_d256(bits_k, bits_v);
}
inline hipError_t launch_decode_mha_rope(const DecodeArgs& a, int bits_k, int bits_v, int nseqs, hipStream_t s) {
    return a.head_dim == 64    ? launch_decode_mha_rope_d64(a, bits_k, bits_v, nseqs, s)
           : a.head_dim == 128 ? launch_decode_mha_rope_d128(a, bits_k, bits_v, nseqs, s)
                               : launch_decode_mha_rope_d256(a, bits_k, bits_v, nseqs, s);
}
hipError_t launch_dequant(const DequantArgs& a, hipStream_t s);
// The library's fixed device scratch (kvq_scratch.hip): its address on the
// current device, taken on the first call there.
constexpr size_t kScratchBytes = 64ull << 20;
hipError_t scratch_address(void** out);
hipError_t launch_decode_window(const DecodeArgs& a, hipStream_t s);
hipError_t launch_read_probe(const void* buf, size_t bytes, uint32_t* sink, hipStream_t s);

// Scatter of 32-bit words: base[index[i]] = value[i], i < count, with the pairs
// in the kernel arguments (no host staging): page-list entries and the
// per-sequence counts of an append.
constexpr int kPageUpdateMax = 480;
struct PageUpdates {
    int32_t count;
    uint32_t index[kPageUpdateMax];
    uint32_t value[kPageUpdateMax];
};
hipError_t launch_page_updates(uint32_t* pages, const PageUpdates& u, hipStream_t s);

}  // namespace kvq
