/*
 * kvq.h — C ABI of libkvq: groupwise asymmetric integer quantization of a
 * transformer KV cache, bit-packed in HBM, and the decode-step attention that
 * reads the packed cache directly (AMD Instinct MI355X, gfx950).
 *
 * Sources, cited by page title and section heading:
 *   [N] nalar.dev, "Kuantisasi KV cache untuk mengurangi memory inferensi
 *       long-context"
 *   [U] unite.ai (pt), "O Seu Cache KV Nao Tem um Problema de Bits. Tem um
 *       Problema de Geometria."
 *   [H] hatterialabs.com (cs), "Asymetrie kvantizace KV cache"
 *
 * The quantizer ([U] "O Que o Erro de Quantizacao E Realmente Feito";
 * [N] "Scale menentukan sistem koordinat kuantisasi"): for every group of
 * values, zero z = group minimum, step s = (max - min) / (2^B - 1) computed in
 * float32 (subtract, then a correctly rounded divide), both stored as fp16
 * (round to nearest even); code = clamp(rint((x - z) / s), 0, 2^B - 1) against
 * the stored z and s, with ties to even; a group whose stored step is 0 gets
 * code 0. Reconstruction is x_hat = z + code * s.
 *
 * Grouping ([U] "Chaves: Os Valores Extremos Vivem em Canais Fixos",
 * "Valores: Onde a Intuicao Quebra"): KVQ_AXIS_CHANNEL keeps one (s, z) per
 * channel for each block of G consecutive tokens (the key default: outlier
 * channels get their own steps); KVQ_AXIS_TOKEN keeps one (s, z) per token for
 * each group of G consecutive channels (the value default: a token's error
 * stays with that token). K and V have separate bit widths B in {2,3,4,6,8}
 * ([N] "Key dan value dapat memiliki struktur numerik berbeda"; [H] "Vychozi
 * zjisteni na GPT-2").
 *
 * Residual ([U] "O Imposto dos Sistemas e Por Que Nao E um Detalhe"; [N]
 * "Pengecualian recent-token mengubah perhitungan memory"): a channel-axis
 * step needs all G tokens of a block, so the last (len mod G) tokens of a
 * channel-axis tensor stay in the input dtype and are quantized when their
 * block completes. Results depend only on the token history, never on how
 * appends were chunked.
 *
 * Storage (the pages leave the layout open: [N] "Scale menentukan ..."):
 *   code row   one token of one head: D/32 units, unit u = B uint32 words
 *              holding channels 32u..32u+31; channel 32u+j sits at bits
 *              [jB, jB+B) of the unit's little-endian bitstream (3- and
 *              6-bit codes straddle words). A row is D*B/8 bytes, no padding.
 *   metadata   uint32 words, fp16 step in bits 0..15, fp16 zero in 16..31;
 *              channel axis: [block][channel]; token axis: [token][group].
 *   residual   channel-axis tensors only: G rows of D input-dtype values per
 *              (layer, seq, head); token t lives in row t mod G.
 *   window     with a window or sinks (kvq_geometry), each tensor's head region
 *              of the residual pool continues (after the G residual rows of a
 *              channel-axis tensor) with sinks + window + block rows of D
 *              input-dtype values: sink token t in row t, later token t in row
 *              sinks + (t mod (window + block)).
 *   pools      four caller-owned device buffers (codes, metadata, residual,
 *              table) sized by kvq_plan; regions are ordered layer -> seq ->
 *              tensor (K, V) -> head, each head region 256-byte aligned.
 *   pages      with kvq_geometry.page_tokens = P > 0 the codes and metadata
 *              live in a shared pool of fixed-size pages instead (the codes
 *              buffer; the metadata buffer is unused). A page holds P
 *              consecutive tokens of one (layer, seq): K code rows [head][P],
 *              V code rows [head][P], then the K and V metadata of those
 *              tokens ([head][P/G][D] on the channel axis, [head][P][D/G] on
 *              the token axis), each head region 256-byte aligned; the page
 *              stride is the largest such size over the cache's bit pairs. A
 *              per-(layer, seq) page list in the table maps logical page i
 *              (tokens iP .. iP + P - 1) to a physical page. Since a key
 *              block never straddles pages, a page carries the steps and
 *              zeros of exactly the codes it holds ([N] "State quantized
 *              cache harus tetap selaras dengan posisi": remapping logical to
 *              physical positions must move the scales with their codes).
 *              Pages are taken from the pool when an append first writes
 *              into them and returned when no sequence refers to them; whole
 *              pages are shared between sequences by reference count
 *              (kvq_gather_sequences). Residual and window rows stay in the
 *              residual pool, per (layer, seq).
 *
 * Conventions
 *   - Every call returns a kvq_status; nothing throws or aborts. On error
 *     nothing is launched, nothing is written and lengths do not advance.
 *     kvq_last_error() gives a detail message for the calling thread.
 *   - The library never allocates device memory. All device buffers belong to
 *     the caller and must stay alive while a cache handle uses them.
 *   - `stream` is a hipStream_t (NULL = the null stream). Calls only enqueue
 *     work on it and return. All calls on one cache must be ordered on one
 *     stream, or synchronized by the caller between streams: the library keeps
 *     the sequence lengths on the host and in the table, and reuses the
 *     table's argument area from call to call.
 *   - One decode step is kvq_quantize_append (the new token) followed by
 *     kvq_decode_attention, which attends to every cached token including
 *     the new one.
 *   - Preconditions on data (not checked on the device): inputs finite and,
 *     with fp16 metadata, |x| <= 65504.
 */
#ifndef KVQ_H
#define KVQ_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef int32_t kvq_status;
#define KVQ_OK               0
#define KVQ_ERR_ARG         -1 /* null pointer, out-of-range index or shape, bad enum      */
#define KVQ_ERR_UNSUPPORTED -2 /* valid request this build does not implement               */
#define KVQ_ERR_CAPACITY    -3 /* an append would exceed a sequence's capacity              */
#define KVQ_ERR_ALIGN       -4 /* a device pointer is not aligned as documented             */
#define KVQ_ERR_WORKSPACE   -5 /* workspace null or smaller than kvq_decode_workspace_size */
#define KVQ_ERR_HIP         -6 /* a HIP runtime call or kernel launch failed                */

enum { KVQ_AXIS_CHANNEL = 0, KVQ_AXIS_TOKEN = 1 };
enum { KVQ_F32 = 0, KVQ_F16 = 1, KVQ_BF16 = 2 };

/* The problem statement ([N] "Ukuran cache bertambah mengikuti token, layer,
 * dan KV head": layers, cached tokens, kv heads, head_dim; [N] "Scale
 * menentukan ...": group size, axis, precision of the scale). */
typedef struct kvq_geometry {
    int32_t layers;     /* >= 1                                                  */
    int32_t num_seqs;   /* >= 1                                                  */
    int32_t kv_heads;   /* >= 1                                                  */
    int32_t q_heads;    /* multiple of kv_heads; head h reads kv head h/(q/kv)   */
    int32_t head_dim;   /* D: multiple of 32, at most 256                        */
    int32_t group_k;    /* G for K: 32, 64, 128 or 256 (token axis: divides D)   */
    int32_t group_v;    /* G for V: same rules                                   */
    int32_t axis_k;     /* KVQ_AXIS_CHANNEL (default for keys)                   */
    int32_t axis_v;     /* KVQ_AXIS_TOKEN   (default for values)                 */
    int32_t in_dtype;   /* KVQ_F32, KVQ_F16 or KVQ_BF16: K/V/q inputs, residual  */
    int32_t meta_dtype; /* KVQ_F16 (the only metadata type this build stores)    */
    /* Full-precision recent window and attention sinks ([U] "O Imposto dos
     * Sistemas ...": the most recent tokens, up to a window of about 128,
     * stay in full precision; [U] "O Que Fazer Com Isso" and "Onde o
     * Trabalho Esta Indo": high-precision windows for recent and sink tokens;
     * [N] "Pengecualian recent-token ...": a high-precision region next to the
     * packed cache). Both 0 (the default): off, only the channel-axis
     * residual above is unquantized. Otherwise the decode attention (and
     * kvq_dequantize) reads a token in the input dtype when t < sinks or when
     * it is not inside a whole key block lying in [sinks, len - window); the
     * blocks inside are read quantized. A block is the token length of a
     * channel-axis group (the larger one when both tensors are on the channel
     * axis; 1 token when neither is). So between window and
     * window + block - 1 recent tokens are full precision. Both tensors share
     * the boundary. Every token is still quantized on arrival (the stored
     * codes do not depend on the window); the full-precision rows are kept
     * besides, in the residual pool. Limits: 0 <= window, 0 <= sinks,
     * sinks a multiple of the key block, sinks + window + block <= 4096. */
    int32_t window;     /* R: recent tokens kept in full precision (0: none)    */
    int32_t sinks;      /* S: first tokens kept in full precision (0: none)     */
    /* Keys cached before the rotary position embedding ([U] "Embebedos
     * Rotatorios Complicam as Chaves": rotation spreads a fixed outlier
     * channel into its partner, so the keys are quantized before it and
     * rotated after dequantization). 0: off. Otherwise the appended keys are
     * taken as un-rotated, and the decode attention rotates the reconstructed
     * key of token t to position t: channel pair (i, i + head_dim/2) turns by
     * t * rope_base^(-2i/head_dim); q must be given rotated to its own
     * position. kvq_dequantize returns the un-rotated keys. With a window or
     * sinks the full-precision rows are rotated to their positions too. This
     * build: channel-axis keys (else KVQ_ERR_UNSUPPORTED at decode); the
     * single-query kernel (head_dim 64, 128, 256) and the query-group kernel
     * (head_dim 128, 256) have rotary instantiations, other caches take the
     * generic split kernel. */
    double rope_base;
    /* Paged storage (see "pages" above). 0: each (layer, seq) has contiguous
     * regions sized for its capacity. Otherwise P tokens per page: a power of
     * two, 64 <= P <= 65536, at least the key block, with sinks a multiple
     * of P. */
    int32_t page_tokens;
    /* Physical pages in the pool (paged storage; 0: enough for every
     * sequence of every layer at full capacity). At most 2^31 - 1. */
    int32_t num_pages;
} kvq_geometry;

/* Byte counts. The pool sizes include 256-byte alignment of every head
 * region; the formula_* fields are the closed-form bytes at full capacity
 * with no padding ([N] "Pengecualian recent-token ...": packed cache +
 * scales/metadata + high-precision recent cache + workspace). */
typedef struct kvq_sizes {
    uint64_t codes_bytes;            /* codes pool                                   */
    uint64_t meta_bytes;             /* metadata pool                                */
    uint64_t residual_bytes;         /* residual pool                                */
    uint64_t table_bytes;            /* table buffer (offsets, lengths, call args)   */
    uint64_t formula_codes_bytes;    /* sum rows * kv_heads * D * B / 8              */
    uint64_t formula_meta_bytes;     /* 4 bytes per group                            */
    uint64_t formula_residual_bytes; /* G * D * in_bytes per channel-axis tensor head,
                                        plus (sinks + window + block) * D * in_bytes per
                                        tensor head with a window or sinks            */
    uint64_t page_bytes;             /* paged storage: stride of a physical page (else 0) */
    uint64_t num_pages;              /* paged storage: pages in the codes pool (else 0)   */
} kvq_sizes;

/* Byte offsets of one (layer, seq) in the pools, head 0, plus per-head
 * strides; for serialization, inspection and tests. With paged storage the
 * codes and metadata offsets and strides are inside a page (kvq_page_list
 * gives the pages); the residual offsets are pool offsets as before. */
typedef struct kvq_region {
    uint64_t k_codes, v_codes, k_meta, v_meta, k_resid, v_resid;
    uint64_t k_codes_head_stride, v_codes_head_stride;
    uint64_t k_meta_head_stride, v_meta_head_stride;
    uint64_t k_resid_head_stride, v_resid_head_stride;
    int32_t bits_k, bits_v, capacity, length;
} kvq_region;

typedef struct kvq_cache kvq_cache;

/* Pool sizes for a geometry. capacity, bits_k, bits_v: host arrays of
 * num_seqs entries (capacity >= 0 tokens per sequence and layer; bits in
 * {2,3,4,6,8}). Pure host computation. */
kvq_status kvq_plan(const kvq_geometry* geometry, const int32_t* capacity,
                    const uint8_t* bits_k, const uint8_t* bits_v, kvq_sizes* out);

/* Create a cache handle over caller-owned device pools (each at least the
 * size kvq_plan reports, 256-byte aligned). Writes the offset table and zero
 * lengths into d_table with a blocking copy on `stream`; pool contents are
 * not touched. The handle is a small host object freed by
 * kvq_cache_destroy. */
kvq_status kvq_cache_create(const kvq_geometry* geometry, const int32_t* capacity,
                            const uint8_t* bits_k, const uint8_t* bits_v,
                            void* d_codes, void* d_meta, void* d_residual, void* d_table,
                            void* stream, kvq_cache** out);

/* Free the host handle (the device pools stay with the caller). NULL is a no-op. */
void kvq_cache_destroy(kvq_cache* cache);

/* Append n_new[s] tokens to every sequence s of `layer` and quantize what
 * becomes quantizable ([U] "O Imposto dos Sistemas ...": token-axis groups
 * at once, channel-axis blocks when their G-th token arrives). k_new, v_new:
 * device, in_dtype, [sum(n_new)][kv_heads][head_dim], sequences in order
 * (element-aligned). n_new: host array of num_seqs counts >= 0. A bulk
 * prefill is an append into an empty cache. Errors: KVQ_ERR_CAPACITY when
 * length + n_new > capacity for any sequence (nothing is written). */
kvq_status kvq_quantize_append(kvq_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                               const int32_t* n_new, void* stream);

/* Bytes of workspace kvq_decode_attention needs for this cache at any
 * length up to capacity (split partials; caller-owned, 256-byte aligned). */
size_t kvq_decode_workspace_size(const kvq_cache* cache);

/* Which decode kernel every decode call on this cache runs (host only; the
 * choice depends on the geometry and the cache's bit pairs, never on the
 * lengths), so that a cache that falls to the generic kernel is visible
 * before it is timed:
 *   KVQ_DECODE_SINGLE_QUERY: one query per kv head (per-channel keys,
 *     per-token values, head_dim 64, 128 or 256);
 *   KVQ_DECODE_QUERY_GROUP: 2 or more query heads per kv head, same caches
 *     (rotary keys: head_dim 128 and 256; head_dim 64: even key bit widths);
 *   KVQ_DECODE_GENERIC: the generic split kernel (every other cache), much
 *     slower.
 * Errors: KVQ_ERR_ARG for a NULL argument; KVQ_ERR_UNSUPPORTED where decode
 * itself fails with it (the generic kernel with more than 16 query heads per
 * kv head, rotary keys on the token axis). */
enum { KVQ_DECODE_SINGLE_QUERY = 1, KVQ_DECODE_QUERY_GROUP = 2, KVQ_DECODE_GENERIC = 3 };
kvq_status kvq_decode_kernel(const kvq_cache* cache, int32_t* kernel);

/* Decode-step attention of one query per sequence and query head over every
 * cached token of `layer`, reading the packed codes and fp16 metadata and
 * dequantizing in registers ([N] "Kuantisasi dapat memindahkan pekerjaan ke
 * decode path": the fused alternative to dequantizing into a temporary;
 * [U] "Por Que o Cache KV E Onde Isso Morde": decode reads the whole cache
 * once per generated token). out[s][h] = sum_t softmax_t(scale * q.k_hat_t) *
 * v_hat_t, keys in the residual taken as stored. q: device, in_dtype,
 * [num_seqs][q_heads][head_dim]; out: device float32, same shape; a sequence
 * of length 0 gets zeros. K and V on either axis. Per-channel keys with
 * per-token values and head_dim 64, 128 or 256 take the single-query or
 * query-group kernel (any q_heads/kv_heads; rotary keys: the query-group
 * kernel at head_dim 128 and 256 only); other caches (per-token keys,
 * per-channel values, other head_dims) take the generic split kernel, which
 * needs q_heads/kv_heads <= 16 (else KVQ_ERR_UNSUPPORTED). */
kvq_status kvq_decode_attention(const kvq_cache* cache, int32_t layer, const void* q, float softmax_scale,
                                float* out, void* workspace, size_t workspace_bytes, void* stream);

/* For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc):
 * kvq_decode_attention with the same arguments minus the workspace, and the
 * same results bit for bit. The split workspace comes from a fixed device
 * array of the library, 64 MiB per GPU, held until the process ends; the call
 * allocates nothing. A call whose workspace would exceed it (about 64 MiB /
 * (4 * (head_dim + 2) * num_seqs * q_heads) splits per sequence) fails with
 * KVQ_ERR_WORKSPACE before anything is launched. Every call on one GPU shares
 * that GPU's array: calls that overlap on one GPU (other streams, other host
 * threads) race and must be ordered by the caller. Other errors as for
 * kvq_decode_attention; KVQ_ERR_HIP if the array's address cannot be taken. */
kvq_status kvq_decode_attention_noalloc(const kvq_cache* cache, int32_t layer, const void* q, float softmax_scale,
                                        float* out, void* stream);

/* One decode step of `layer`: kvq_quantize_append(k_new, v_new, n_new) then
 * kvq_decode_attention(q), with the same arguments, results and errors (all
 * checked before anything is launched or written). Where the single-query
 * kernel serves the cache (q_heads == kv_heads, keys per channel, values per
 * token) and the step completes no key block and adds at most
 * 256 / (head_dim / 32) rows per sequence, both run in one launch: each
 * (sequence, kv head) workgroup that attends the newest tokens first appends
 * them, and with a window or sinks also copies them into the window area
 * (for bit pairs where the fused kernel keeps the plain one's occupancy).
 * Otherwise the two run as consecutive launches. */
kvq_status kvq_decode_step(kvq_cache* cache, int32_t layer, const void* k_new, const void* v_new,
                           const int32_t* n_new, const void* q, float softmax_scale, float* out, void* workspace,
                           size_t workspace_bytes, void* stream);

/* kvq_quantize_append of the same per-sequence counts n_new into each of the
 * n_layers consecutive layers [layer0, layer0 + n_layers), in one launch: the
 * append of a whole model's decode step. k_new, v_new: device, in_dtype,
 * [n_layers][sum n_new][kv_heads][head_dim] (layer layer0 + i takes slice i).
 * The stored bytes equal n_layers single-layer appends. 1 <= n_layers <= 64
 * (more: KVQ_ERR_UNSUPPORTED); capacity is checked for every layer and
 * sequence before anything is written (KVQ_ERR_CAPACITY); other errors as
 * for kvq_quantize_append. */
kvq_status kvq_quantize_append_layers(kvq_cache* cache, int32_t layer0, int32_t n_layers, const void* k_new,
                                      const void* v_new, const int32_t* n_new, void* stream);

/* kvq_decode_attention for the n_layers consecutive layers [layer0, layer0 +
 * n_layers) in one call whose kernels each cover all of them: the decode step
 * of a whole model whose per-layer caches are too small to fill the GPU alone.
 * Layer layer0 + i reads q + i * num_seqs * q_heads * head_dim elements and
 * writes out + i * num_seqs * q_heads * head_dim floats; the results equal n_layers
 * single-layer calls up to the summation order of split partials. workspace:
 * at least n_layers * kvq_decode_workspace_size(cache) bytes, 256-byte aligned.
 * 1 <= n_layers <= 64 (more: KVQ_ERR_UNSUPPORTED); other errors as for
 * kvq_decode_attention, checked before any launch. */
kvq_status kvq_decode_attention_layers(const kvq_cache* cache, int32_t layer0, int32_t n_layers, const void* q,
                                       float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                                       void* stream);

/* The unfused path ([N] "Kuantisasi dapat memindahkan pekerjaan ke decode
 * path": dequantize into a temporary floating-point tensor): write x_hat =
 * fma(code, s, z) in float32 for every cached token of one sequence, residual
 * rows converted exactly from the input dtype. k_out, v_out: device float32
 * [kv_heads][length][head_dim] (either may be NULL to skip it). */
kvq_status kvq_dequantize(const kvq_cache* cache, int32_t layer, int32_t seq, float* k_out, float* v_out,
                          void* stream);

/* Measurement aid, not part of the method: read `bytes` (a multiple of 16)
 * of device memory at `buf` (16-byte aligned) with the plainest streaming
 * loop, so that a caller can time the HBM read ceiling the decode kernels are
 * compared with. Nothing is written except possibly one word at `sink`
 * (device, 4-byte aligned). bytes == 0 is a no-op. Errors: KVQ_ERR_ARG (NULL
 * pointer, size not a multiple of 16), KVQ_ERR_ALIGN, KVQ_ERR_HIP. */
kvq_status kvq_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* stream);

/* Copy sequence src_seq of `src` over sequence dst_seq of `dst`, for layers
 * [layer0, layer0 + n_layers): its packed codes, metadata, residual rows,
 * window rows and length, so that dst_seq then decodes exactly as src_seq
 * (beam forks, prefix reuse: [N] "State quantized cache harus tetap selaras
 * dengan posisi": the scales and packing metadata must move with the codes
 * they describe). `dst` and `src` may be the same cache (then dst_seq !=
 * src_seq). Requires equal geometry (every kvq_geometry field) and, for the
 * two sequences, equal bits_k, bits_v and capacity. Device-to-device copies
 * enqueued on `stream`; only the bytes of the first `length` tokens are
 * defined afterwards. Paged storage: dst must be src, and the copy is
 * kvq_gather_sequences with src[dst_seq] = src_seq (shared pages). Errors:
 * KVQ_ERR_ARG (NULL cache, index out of range, mismatch, same sequence),
 * KVQ_ERR_UNSUPPORTED (paged storage across two caches), KVQ_ERR_CAPACITY
 * (paged: no free page), KVQ_ERR_HIP. */
kvq_status kvq_copy_sequence(kvq_cache* dst, int32_t dst_seq, const kvq_cache* src, int32_t src_seq, int32_t layer0,
                             int32_t n_layers, void* stream);

/* Reorder and fork sequences ([N] "State quantized cache harus tetap selaras
 * dengan posisi": beam operations and prefix reuse remap logical to physical
 * slots, and the scales must move with the codes they describe): afterwards
 * sequence s of each layer in [layer0, layer0 + n_layers) holds what sequence
 * src[s] held before the call (codes, metadata, residual and window rows,
 * length), for every s at once. src: host array of num_seqs indices; src[s]
 * == s leaves s as it is, and an index may appear several times (beam
 * search: surviving beams replace dropped ones; prefix sharing: one prompt's
 * cache forked into several sequences). s and src[s] must have equal bits_k,
 * bits_v and capacity. Paged storage: whole pages are shared by reference
 * count, only the page holding a source's last incomplete page of tokens is
 * copied, once per extra copy; contiguous storage: the regions of extra
 * copies are copied into the regions of sequences no one refers to. Copies
 * and table updates are enqueued on `stream`. Errors: KVQ_ERR_ARG (NULL,
 * index out of range, mismatched bits or capacity), KVQ_ERR_CAPACITY (paged:
 * not enough free pages; nothing changes), KVQ_ERR_HIP. */
kvq_status kvq_gather_sequences(kvq_cache* cache, int32_t layer0, int32_t n_layers, const int32_t* src, void* stream);

/* Evict tokens [first, first + count) of sequence `seq` in layers [layer0,
 * layer0 + n_layers) ([N] "State quantized cache harus tetap selaras dengan
 * posisi": eviction remaps logical positions; the pages go with their own
 * steps and zeros). Paged storage only: first and count multiples of
 * page_tokens, first >= sinks, first + count <= the sequence's whole pages
 * and, with a window, <= length - (window + key block) (the window rows stay
 * valid). The pages are released and later tokens move down by count
 * (keys cached before the rotary embedding are then rotated to their new
 * positions). count == 0 is a no-op. Errors: KVQ_ERR_ARG, KVQ_ERR_UNSUPPORTED
 * (contiguous storage), KVQ_ERR_HIP. */
kvq_status kvq_evict_tokens(kvq_cache* cache, int32_t layer0, int32_t n_layers, int32_t seq, int32_t first,
                            int32_t count, void* stream);

/* Empty sequence `seq` in layers [layer0, layer0 + n_layers): length 0, and
 * with paged storage its pages released. Errors: KVQ_ERR_ARG, KVQ_ERR_HIP. */
kvq_status kvq_reset_sequence(kvq_cache* cache, int32_t layer0, int32_t n_layers, int32_t seq, void* stream);

/* Physical page of each logical page of (layer, seq), paged storage (host
 * array of up to max_out entries; 0xFFFFFFFF = no page), and the number of
 * logical pages the sequence's capacity spans in *n_pages. free_pages (may be
 * NULL): pages of the pool no sequence refers to. Errors: KVQ_ERR_ARG,
 * KVQ_ERR_UNSUPPORTED (contiguous storage). */
kvq_status kvq_page_list(const kvq_cache* cache, int32_t layer, int32_t seq, uint32_t* out, int32_t max_out,
                         int32_t* n_pages, int64_t* free_pages);

/* Current cached lengths of `layer`: host array of num_seqs entries. */
kvq_status kvq_seq_lengths(const kvq_cache* cache, int32_t layer, int32_t* out);

/* Pool offsets of one (layer, seq). */
kvq_status kvq_get_region(const kvq_cache* cache, int32_t layer, int32_t seq, kvq_region* out);

/* Static description of a status code; never NULL. */
const char* kvq_status_string(kvq_status status);

/* Detail message of the last failing call on this thread ("" if none). */
const char* kvq_last_error(void);

/* Library version, "major.minor.patch". */
const char* kvq_version(void);

#ifdef __cplusplus
}
#endif

#endif /* KVQ_H */
