// Host side of libkvq: argument validation, pool layout, the per-layer length
// state and kernel launches behind the C ABI declared in include/kvq.h.
#include "kvq.h"

#include <hip/hip_runtime_api.h>

#include <algorithm>
#include <cmath>
#include <cstdarg>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <new>
#include <string>
#include <vector>

#include "kvq_internal.h"

namespace kvq {
size_t decode_lds_bytes(int R, int D, int C);
}

using kvq::SeqEntry;

struct kvq_cache {
    kvq_geometry g{};
    std::vector<int32_t> cap;
    std::vector<uint8_t> bits_k, bits_v;
    uint8_t* codes = nullptr;
    uint8_t* meta = nullptr;
    uint8_t* resid = nullptr;
    uint8_t* table = nullptr;
    kvq::TableLayout tl{};
    std::vector<SeqEntry> entries;  // [layers][num_seqs], as on the device
    // Regions of each slot ([layers][num_seqs]): the residual (and, with
    // contiguous storage, code and metadata) regions laid out for sequence i
    // at creation. A sequence uses the regions of slot[l][s], which
    // kvq_gather_sequences remaps so that a reorder copies only extra copies.
    std::vector<SeqEntry> slot_layout;
    std::vector<int32_t> slot;
    // Paged storage: the pool's free pages (a stack), the references to each
    // page, and the host copy of the device page lists.
    bool paged = false;
    uint64_t page_bytes = 0;
    uint32_t num_pages = 0;
    std::vector<uint32_t> free_pages;
    std::vector<uint32_t> refs;
    std::vector<uint32_t> pt;
    std::vector<int32_t> lens;      // host mirror of the current lengths [layers][num_seqs]
    std::vector<uint8_t> parity;    // which length buffer is current, per layer
    struct Pair { int bk, bv, offset, count; };
    std::vector<Pair> pairs;        // distinct (bits_k, bits_v) pairs and their slice of the table's seq list
    std::vector<int32_t> pair_list; // host copy of that seq list
    int32_t max_cap = 0;
};

namespace {

thread_local std::string g_last_error;

kvq_status fail(kvq_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
kvq_status fail(kvq_status st, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof buf, fmt, ap);
    va_end(ap);
    g_last_error = buf;
    return st;
}

kvq_status hip_fail(hipError_t e, const char* what) {
    return fail(KVQ_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

uint64_t align_up(uint64_t x, uint64_t a) { return (x + a - 1) / a * a; }

int in_bytes(int dt) { return dt == KVQ_F32 ? 4 : 2; }

bool valid_bits(int b) { return b == 2 || b == 3 || b == 4 || b == 6 || b == 8; }

bool aligned(const void* p, uint64_t a) { return ((uintptr_t)p % a) == 0; }

// Full-precision window and sinks: on when either is non-zero.
bool win_mode(const kvq_geometry& g) { return g.window != 0 || g.sinks != 0; }

// Token length of a key block: the larger channel-axis group, 1 when no tensor
// groups along tokens.
int token_block(const kvq_geometry& g) {
    int b = 1;
    if (g.axis_k == KVQ_AXIS_CHANNEL) b = std::max(b, g.group_k);
    if (g.axis_v == KVQ_AXIS_CHANNEL) b = std::max(b, g.group_v);
    return b;
}

// Rows of the window area per (tensor, head): the sinks, then a ring of
// window + block rows for the recent tokens.
int win_rows(const kvq_geometry& g) { return g.window + token_block(g); }

// Byte offset of the window area inside tensor t's head region of the residual
// pool (after the G residual rows of a channel-axis tensor).
uint32_t win_off(const kvq_geometry& g, int t) {
    const int axis = t == 0 ? g.axis_k : g.axis_v, G = t == 0 ? g.group_k : g.group_v;
    return axis == KVQ_AXIS_CHANNEL ? (uint32_t)((uint64_t)G * g.head_dim * in_bytes(g.in_dtype)) : 0u;
}

kvq_status check_geometry(const kvq_geometry* g) {
    if (!g) return fail(KVQ_ERR_ARG, "geometry is NULL");
    if (g->layers < 1 || g->num_seqs < 1 || g->kv_heads < 1 || g->q_heads < 1)
        return fail(KVQ_ERR_ARG, "layers, num_seqs, kv_heads and q_heads must be >= 1");
    if (g->q_heads % g->kv_heads)
        return fail(KVQ_ERR_ARG, "q_heads (%d) is not a multiple of kv_heads (%d)", g->q_heads, g->kv_heads);
    if (g->head_dim < 32 || g->head_dim % 32 || g->head_dim > kvq::kMaxHeadDim)
        return fail(KVQ_ERR_ARG, "head_dim (%d) must be a multiple of 32 in [32, 256]", g->head_dim);
    const int groups[2] = {g->group_k, g->group_v};
    const int axes[2] = {g->axis_k, g->axis_v};
    for (int t = 0; t < 2; ++t) {
        const int G = groups[t];
        if (G != 32 && G != 64 && G != 128 && G != 256)
            return fail(KVQ_ERR_ARG, "group_%c (%d) must be 32, 64, 128 or 256", "kv"[t], G);
        if (axes[t] != KVQ_AXIS_CHANNEL && axes[t] != KVQ_AXIS_TOKEN)
            return fail(KVQ_ERR_ARG, "axis_%c (%d) is not a kvq axis", "kv"[t], axes[t]);
        if (axes[t] == KVQ_AXIS_TOKEN && g->head_dim % G)
            return fail(KVQ_ERR_ARG, "token-axis group_%c (%d) must divide head_dim (%d)", "kv"[t], G, g->head_dim);
    }
    if (g->in_dtype != KVQ_F32 && g->in_dtype != KVQ_F16 && g->in_dtype != KVQ_BF16)
        return fail(KVQ_ERR_ARG, "in_dtype (%d) is not a kvq dtype", g->in_dtype);
    if (g->meta_dtype == KVQ_F32 || g->meta_dtype == KVQ_BF16)
        return fail(KVQ_ERR_UNSUPPORTED, "only fp16 step/zero metadata is stored by this build");
    if (g->meta_dtype != KVQ_F16) return fail(KVQ_ERR_ARG, "meta_dtype (%d) is not a kvq dtype", g->meta_dtype);
    if (g->window < 0 || g->sinks < 0) return fail(KVQ_ERR_ARG, "window (%d) and sinks (%d) must be >= 0", g->window, g->sinks);
    if (!(g->rope_base >= 0.0) || g->rope_base > 1e30) return fail(KVQ_ERR_ARG, "rope_base must be finite and >= 0");
    if (g->rope_base > 0.0 && g->rope_base <= 1.0) return fail(KVQ_ERR_ARG, "rope_base must be > 1 (or 0: off)");
    if (win_mode(*g)) {
        const int b = token_block(*g);
        if (g->sinks % b) return fail(KVQ_ERR_ARG, "sinks (%d) must be a multiple of the key block (%d tokens)", g->sinks, b);
        if ((long)g->sinks + g->window + b > 4096)
            return fail(KVQ_ERR_ARG, "sinks + window + block = %ld exceeds 4096", (long)g->sinks + g->window + b);
    }
    if (g->page_tokens < 0 || g->num_pages < 0)
        return fail(KVQ_ERR_ARG, "page_tokens (%d) and num_pages (%d) must be >= 0", g->page_tokens, g->num_pages);
    if (g->page_tokens) {
        const int P = g->page_tokens;
        if (P < 64 || P > 65536 || (P & (P - 1)))
            return fail(KVQ_ERR_ARG, "page_tokens (%d) must be a power of two in [64, 65536]", P);
        if (P < token_block(*g))
            return fail(KVQ_ERR_ARG, "page_tokens (%d) must be at least the key block (%d tokens)", P, token_block(*g));
        if (g->sinks % P) return fail(KVQ_ERR_ARG, "sinks (%d) must be a multiple of page_tokens (%d)", g->sinks, P);
    }
    return KVQ_OK;
}

kvq_status check_seqs(const kvq_geometry* g, const int32_t* cap, const uint8_t* bk, const uint8_t* bv) {
    if (!cap || !bk || !bv) return fail(KVQ_ERR_ARG, "capacity, bits_k and bits_v must be non-NULL");
    for (int s = 0; s < g->num_seqs; ++s) {
        if (cap[s] < 0 || cap[s] > (1 << 28)) return fail(KVQ_ERR_ARG, "capacity[%d] = %d out of range", s, cap[s]);
        if (!valid_bits(bk[s]) || !valid_bits(bv[s]))
            return fail(KVQ_ERR_ARG, "bits of sequence %d (%d, %d) must be in {2,3,4,6,8}", s, bk[s], bv[s]);
    }
    return KVQ_OK;
}

// Logical pages of a sequence of capacity cap (paged storage).
uint32_t pages_of(const kvq_geometry* g, int cap) {
    return (uint32_t)(((int64_t)cap + g->page_tokens - 1) / g->page_tokens);
}

// Pool layout. Contiguous storage: layer -> seq -> tensor (K, V) -> head, each
// head region 256-byte aligned. Paged storage: codes and metadata inside a page
// (K codes, V codes, K metadata, V metadata, each [head] with 256-byte aligned
// head regions; the page stride is the largest over the sequences), residual
// regions as with contiguous storage. Fails when the pool would not be
// addressable (page lists or page indices beyond 32 bits).
// Rotary tables of a cache with rope_base > 0 (device copy in the table
// buffer): theta_i = base^(-2i/D) for the D/2 pairs (i, i + D/2) as doubles,
// then (cos, sin)(u theta_i) as floats for u = 0..kRopeRows-1, row-major
// [u][i] ([U] "Embebedos Rotatorios Complicam as Chaves").
uint64_t rope_table_bytes(int head_dim) {
    return (uint64_t)head_dim / 2 * 8 + (uint64_t)kvq::kRopeRows * head_dim / 2 * 8;
}
void fill_rope_tables(const kvq_geometry& g, uint8_t* dst) {
    const int P = g.head_dim / 2;
    double* theta = (double*)dst;
    float* tab = (float*)(dst + (size_t)P * 8);
    for (int i = 0; i < P; ++i) theta[i] = std::pow(g.rope_base, -2.0 * i / g.head_dim);
    for (int u = 0; u < kvq::kRopeRows; ++u)
        for (int i = 0; i < P; ++i) {
            const double ang = u * theta[i];
            tab[2 * ((size_t)u * P + i)] = (float)std::cos(ang);
            tab[2 * ((size_t)u * P + i) + 1] = (float)std::sin(ang);
        }
}

kvq_status layout(const kvq_geometry* g, const int32_t* cap, const uint8_t* bk, const uint8_t* bv,
                  std::vector<SeqEntry>* entries, kvq_sizes* sz, kvq::TableLayout* tl) {
    const uint64_t D = g->head_dim, H = g->kv_heads, ib = in_bytes(g->in_dtype);
    const int groups[2] = {g->group_k, g->group_v};
    const int axes[2] = {g->axis_k, g->axis_v};
    const bool paged = g->page_tokens > 0;
    const uint64_t P = paged ? (uint64_t)g->page_tokens : 0;
    uint64_t oc = 0, om = 0, orr = 0, fc = 0, fm = 0, fr = 0, page_bytes = 0, plist = 0;
    if (entries) entries->assign((size_t)g->layers * g->num_seqs, SeqEntry{});
    for (int l = 0; l < g->layers; ++l) {
        for (int s = 0; s < g->num_seqs; ++s) {
            SeqEntry e{};
            const int bits[2] = {bk[s], bv[s]};
            uint64_t in_page = 0;  // paged: bytes of this sequence's page
            for (int t = 0; t < 2; ++t) {
                const uint64_t G = groups[t], B = bits[t], c = cap[s];
                const bool ch = axes[t] == KVQ_AXIS_CHANNEL;
                const uint64_t rows = ch ? (c / G) * G : c;
                const uint64_t code_b = rows * D * B / 8;
                const uint64_t meta_b = (ch ? (c / G) * D : c * (D / G)) * 4;
                const uint64_t res_b = (ch ? G * D * ib : 0) +
                                       (win_mode(*g) ? (uint64_t)(g->sinks + win_rows(*g)) * D * ib : 0);
                if (paged) {
                    e.codes_hs[t] = align_up(P * D * B / 8, kvq::kAlign);
                    e.meta_hs[t] = align_up((ch ? (P / G) * D : P * (D / G)) * 4, kvq::kAlign);
                } else {
                    e.codes[t] = oc;
                    e.codes_hs[t] = align_up(code_b, kvq::kAlign);
                    oc += e.codes_hs[t] * H;
                    e.meta[t] = om;
                    e.meta_hs[t] = align_up(meta_b, kvq::kAlign);
                    om += e.meta_hs[t] * H;
                }
                e.resid[t] = orr;
                e.resid_hs[t] = align_up(res_b, kvq::kAlign);
                orr += e.resid_hs[t] * H;
                fc += code_b * H;
                fm += meta_b * H;
                fr += res_b * H;
                e.bits[t] = bits[t];
            }
            if (paged) {
                e.codes[0] = 0;
                e.codes[1] = e.codes_hs[0] * H;
                e.meta[0] = e.codes[1] + e.codes_hs[1] * H;
                e.meta[1] = e.meta[0] + e.meta_hs[0] * H;
                in_page = e.meta[1] + e.meta_hs[1] * H;
                page_bytes = std::max(page_bytes, in_page);
                e.page_shift = __builtin_ctz((unsigned)g->page_tokens);
                e.page_list = (uint32_t)plist;
                plist += pages_of(g, cap[s]);
                if (plist > 0xffffffffull) return fail(KVQ_ERR_ARG, "page lists exceed 2^32 entries");
            } else {
                e.page_shift = kvq::kContiguousShift;
                e.page_list = 0;
            }
            e.cap = cap[s];
            if (entries) (*entries)[(size_t)l * g->num_seqs + s] = e;
        }
    }
    uint64_t num_pages = 0;
    if (paged) {
        num_pages = g->num_pages ? (uint64_t)g->num_pages : plist;
        if (num_pages >= kvq::kNoPage) return fail(KVQ_ERR_ARG, "%llu pages exceed the page index range",
                                                   (unsigned long long)num_pages);
        if (entries)
            for (auto& e : *entries) e.page_bytes = page_bytes;
        oc = num_pages * page_bytes;
        om = 0;
    }
    const uint64_t LS = (uint64_t)g->layers * g->num_seqs;
    tl->entries_bytes = align_up(LS * sizeof(SeqEntry), kvq::kAlign);
    tl->len_off = tl->entries_bytes;
    tl->args_off = tl->len_off + align_up(2 * LS * 4, kvq::kAlign);
    tl->ctr_off = tl->args_off + align_up(2 * (uint64_t)g->num_seqs * 4, kvq::kAlign);
    tl->pairs_off = tl->ctr_off + align_up((uint64_t)g->num_seqs * g->kv_heads * 4, kvq::kAlign);
    tl->pt_off = tl->pairs_off + align_up((uint64_t)g->num_seqs * 4, kvq::kAlign);
    tl->rope_off = tl->pt_off + align_up(std::max<uint64_t>(plist, 1) * 4, kvq::kAlign);
    tl->total = tl->rope_off + (g->rope_base > 0.0 ? align_up(rope_table_bytes(g->head_dim), kvq::kAlign) : 0);
    sz->codes_bytes = std::max<uint64_t>(oc, kvq::kAlign);
    sz->meta_bytes = std::max<uint64_t>(om, kvq::kAlign);
    sz->residual_bytes = std::max<uint64_t>(orr, kvq::kAlign);
    sz->table_bytes = tl->total;
    sz->formula_codes_bytes = fc;
    sz->formula_meta_bytes = fm;
    sz->formula_residual_bytes = fr;
    sz->page_bytes = page_bytes;
    sz->num_pages = num_pages;
    return KVQ_OK;
}

int group_size(const kvq_cache* c) { return c->g.q_heads / c->g.kv_heads; }

// The buffer the kernels read metadata from: the page pool with paged storage.
uint8_t* meta_pool(const kvq_cache* c) { return c->paged ? c->codes : c->meta; }

const uint32_t* page_lists(const kvq_cache* c) { return (const uint32_t*)(c->table + c->tl.pt_off); }

// Tokens per decode split: a multiple of the key block, grown while the grid
// stays above ~8 workgroups per compute unit, shrunk to fit 64 KB of LDS.
int choose_chunk(const kvq_cache* c, int max_len, int n_layers) {
    const kvq_geometry& g = c->g;
    const int kmin = g.axis_k == KVQ_AXIS_CHANNEL ? std::max(64, g.group_k) : 64;
    const long pairs = (long)g.num_seqs * g.kv_heads * n_layers;
    if (const char* env = std::getenv("KVQ_DECODE_CHUNK")) {  // tuning override, ignored when invalid
        const int v = std::atoi(env);
        if (v >= kmin && v <= 1024 && v % kmin == 0 && (v & (v - 1)) == 0 &&
            kvq::decode_lds_bytes(group_size(c), g.head_dim, v) <= 65536)
            return v;
    }
    int C = kmin;
    while (C < 1024 && pairs * ((max_len + 2L * C - 1) / (2L * C)) >= 2048) C *= 2;
    while (C > kmin && kvq::decode_lds_bytes(group_size(c), g.head_dim, C) > 65536) C /= 2;
    return C;
}

// Tokens per workgroup of the single-query kernel: a multiple of 64 and of the
// key block; a sequence of length L gets
// max(1, L / chunk) splits, the last one taking the remainder.
int choose_split_mha(const kvq_cache* c, int max_len, int n_layers) {
    const kvq_geometry& g = c->g;
    const int unit = std::max(64, g.group_k);
    // paged storage: a split spans at most 64 of a wave's super-tiles (the page
    // entries the kernel keeps in one register); the last split takes up to
    // twice the chunk
    const long cap = c->paged ? 4096 : (1L << 24);
    if (const char* env = std::getenv("KVQ_DECODE_CHUNK")) {  // tuning override, ignored when invalid
        const int v = std::atoi(env);
        if (v >= unit && v % unit == 0 && v <= cap) return v;
    }
    // Aim at ~512 workgroups (two 4-wave workgroups per compute unit, resident
    // at once): long waves keep per-wave setup and the split merge small.
    const long pairs = (long)g.num_seqs * g.kv_heads * n_layers;
    const long nsplit = std::max(1L, 512L / pairs);
    const long cw = (max_len / nsplit) / unit * unit;
    return (int)std::min(cap, std::max<long>(unit, cw));
}

// Tokens per workgroup of the query-group kernel (a multiple of 128, at least
// 512). One launch over every bit pair (one per pair for batches beyond the
// work list's size). A launch holds gqa_resident_per_cu workgroups per compute
// unit (4 waves each, one per SIMD) and dispatches the rest as slots free up.
// Each workgroup costs its tokens plus a fixed 512 (loading the queries,
// merging the waves, writing a split partial that the merge reads back). A
// launch whose workgroups all fit at once takes its longest one; a larger one
// takes its total cost over the slots plus half its longest workgroup (the
// tail), so a ragged batch is not charged full rounds for its short splits.
// The choice minimises the sum over launches.
// lens: [n_layers][num_seqs], the layers of one launch.
int choose_split_gqa(const kvq_cache* c, const int32_t* lens, int n_layers) {
    const kvq_geometry& g = c->g;
    if (const char* env = std::getenv("KVQ_DECODE_CHUNK")) {  // tuning override, ignored when invalid
        const int v = std::atoi(env);
        // (paged storage: at most 8192, 64 of a wave's tiles, whose page entries the kernel keeps in one register)
        if (v >= 128 && v % 128 == 0 && v <= (c->paged ? 8192 : (1 << 24))) return v;
    }
    const double slots = 256.0 * kvq::gqa_resident_per_cu(g.head_dim, g.rope_base > 0.0);
    const bool one_launch = (long)n_layers * g.num_seqs <= kvq::kGqaListMax;
    const long rows = (long)g.kv_heads * ((group_size(c) + 15) / 16);  // workgroups per split of a sequence
    constexpr double kFixed = 512.0;  // per-workgroup cost in tokens (queries, wave merge, the partial)
    // a launch's time in tokens: all of its workgroups resident at once, the
    // longest; else its work spread over the resident slots (dynamic dispatch)
    // plus half the longest workgroup for the tail
    auto launch = [&](double wgs, double work, double longest) {
        return wgs <= slots ? longest : work / slots + 0.5 * longest;
    };
    double best_cost = -1.0;
    int best = 512;
    for (int cw : {512, 640, 768, 896, 1024, 1280, 1536, 2048, 2560, 3072, 4096, 6144, 8192}) {
        double cost = 0.0, all_wgs = 0.0, all_work = 0.0, all_longest = 0.0;
        for (const auto& pr : c->pairs) {
            double wgs = 0.0, work = 0.0, longest = 0.0;
            for (int l = 0; l < n_layers; ++l)
                for (int i = 0; i < pr.count; ++i) {
                    const long len = lens[(size_t)l * g.num_seqs + c->pair_list[pr.offset + i]];
                    const long n = (len + cw - 1) / cw;
                    wgs += (double)(n * rows);
                    work += (double)((len + n * (long)kFixed) * rows);
                    if (n) longest = std::max(longest, (double)std::min<long>(len, cw) + kFixed);
                }
            cost += wgs ? launch(wgs, work, longest) : 0.0;
            all_wgs += wgs, all_work += work, all_longest = std::max(all_longest, longest);
        }
        if (one_launch) cost = all_wgs ? launch(all_wgs, all_work, all_longest) : 0.0;
        if (best_cost < 0.0 || cost < best_cost) best_cost = cost, best = cw;
    }
    return best;
}

// The decode kernel every call on a cache takes: the single-query and
// query-group kernels for per-channel keys with per-token values at head_dim
// 64, 128 and 256 (rotary keys: the query-group one at head_dim 128 and 256;
// head_dim 64: even key bit widths only, a lane group's half unit of key codes
// being whole words), the generic split kernel otherwise.
int32_t decode_route(const kvq_cache* c) {
    const kvq_geometry& g = c->g;
    const bool rope = g.rope_base > 0.0;
    if (g.axis_k != KVQ_AXIS_CHANNEL || g.axis_v != KVQ_AXIS_TOKEN || !kvq::mha_supported(g.head_dim))
        return KVQ_DECODE_GENERIC;
    if (group_size(c) == 1) return KVQ_DECODE_SINGLE_QUERY;
    if (rope && !kvq::gqa_rope_supported(g.head_dim)) return KVQ_DECODE_GENERIC;
    for (const auto& pr : c->pairs)
        if (g.head_dim < 128 && pr.bk % 2 != 0) return KVQ_DECODE_GENERIC;
    return KVQ_DECODE_QUERY_GROUP;
}

int min_chunk(const kvq_cache* c) {
    return c->g.axis_k == KVQ_AXIS_CHANNEL ? std::max(64, c->g.group_k) : 64;
}

// Workgroups of the full-precision window kernel per (seq, kv head): enough for
// the most full-precision tokens a sequence can have (sinks + window + block - 1).
int win_splits(const kvq_cache* c) {
    if (!win_mode(c->g)) return 0;
    return (c->g.sinks + win_rows(c->g) - 1 + kvq::kWinTokens - 1) / kvq::kWinTokens;
}

}  // namespace

extern "C" {

const char* kvq_version(void) { return "0.1.0"; }

const char* kvq_status_string(kvq_status s) {
    switch (s) {
        case KVQ_OK: return "ok";
        case KVQ_ERR_ARG: return "invalid argument";
        case KVQ_ERR_UNSUPPORTED: return "unsupported by this build";
        case KVQ_ERR_CAPACITY: return "capacity exceeded";
        case KVQ_ERR_ALIGN: return "misaligned device pointer";
        case KVQ_ERR_WORKSPACE: return "workspace missing or too small";
        case KVQ_ERR_HIP: return "HIP runtime error";
        default: return "unknown status";
    }
}

const char* kvq_last_error(void) { return g_last_error.c_str(); }

kvq_status kvq_plan(const kvq_geometry* g, const int32_t* cap, const uint8_t* bk, const uint8_t* bv, kvq_sizes* out) {
    g_last_error.clear();
    kvq_status st = check_geometry(g);
    if (st) return st;
    if ((st = check_seqs(g, cap, bk, bv))) return st;
    if (!out) return fail(KVQ_ERR_ARG, "out is NULL");
    kvq::TableLayout tl;
    return layout(g, cap, bk, bv, nullptr, out, &tl);
}

kvq_status kvq_cache_create(const kvq_geometry* g, const int32_t* cap, const uint8_t* bk, const uint8_t* bv,
                            void* d_codes, void* d_meta, void* d_residual, void* d_table, void* stream,
                            kvq_cache** out) {
    g_last_error.clear();
    kvq_status st = check_geometry(g);
    if (st) return st;
    if ((st = check_seqs(g, cap, bk, bv))) return st;
    if (!out) return fail(KVQ_ERR_ARG, "out is NULL");
    *out = nullptr;
    if (!d_codes || !d_meta || !d_residual || !d_table) return fail(KVQ_ERR_ARG, "a device pool is NULL");
    if (!aligned(d_codes, kvq::kAlign) || !aligned(d_meta, kvq::kAlign) || !aligned(d_residual, kvq::kAlign) ||
        !aligned(d_table, kvq::kAlign))
        return fail(KVQ_ERR_ALIGN, "device pools must be 256-byte aligned");
    kvq_cache* c = new (std::nothrow) kvq_cache;
    if (!c) return fail(KVQ_ERR_ARG, "out of host memory");
    c->g = *g;
    c->cap.assign(cap, cap + g->num_seqs);
    c->bits_k.assign(bk, bk + g->num_seqs);
    c->bits_v.assign(bv, bv + g->num_seqs);
    c->codes = (uint8_t*)d_codes;
    c->meta = (uint8_t*)d_meta;
    c->resid = (uint8_t*)d_residual;
    c->table = (uint8_t*)d_table;
    kvq_sizes sz;
    if ((st = layout(g, cap, bk, bv, &c->entries, &sz, &c->tl))) {
        delete c;
        return st;
    }
    c->slot_layout = c->entries;
    c->slot.resize((size_t)g->layers * g->num_seqs);
    for (size_t i = 0; i < c->slot.size(); ++i) c->slot[i] = (int32_t)(i % g->num_seqs);
    c->paged = g->page_tokens > 0;
    if (c->paged) {
        c->page_bytes = sz.page_bytes;
        c->num_pages = (uint32_t)sz.num_pages;
        c->refs.assign(c->num_pages, 0);
        c->free_pages.resize(c->num_pages);
        for (uint32_t i = 0; i < c->num_pages; ++i) c->free_pages[i] = c->num_pages - 1 - i;  // page 0 on top
        const SeqEntry& last = c->entries.back();
        c->pt.assign((size_t)last.page_list + pages_of(g, last.cap), kvq::kNoPage);
    } else {
        c->pt.assign(1, 0u);
    }
    c->lens.assign((size_t)g->layers * g->num_seqs, 0);
    c->parity.assign(g->layers, 0);
    c->max_cap = *std::max_element(cap, cap + g->num_seqs);
    std::vector<uint8_t> img(c->tl.total, 0);
    std::memcpy(img.data(), c->entries.data(), c->entries.size() * sizeof(SeqEntry));
    std::memcpy(img.data() + c->tl.pt_off, c->pt.data(), c->pt.size() * sizeof(uint32_t));
    if (g->rope_base > 0.0) fill_rope_tables(*g, img.data() + c->tl.rope_off);
    {
        int32_t* list = (int32_t*)(img.data() + c->tl.pairs_off);
        int n = 0;
        for (int bkk : {2, 3, 4, 6, 8})
            for (int bvv : {2, 3, 4, 6, 8}) {
                const int start = n;
                for (int s2 = 0; s2 < g->num_seqs; ++s2)
                    if (bk[s2] == bkk && bv[s2] == bvv) list[n++] = s2;
                if (n > start) c->pairs.push_back({bkk, bvv, start, n - start});
            }
        c->pair_list.assign(list, list + n);
    }
    hipStream_t s = (hipStream_t)stream;
    hipError_t e = hipMemcpyAsync(d_table, img.data(), img.size(), hipMemcpyHostToDevice, s);
    if (e == hipSuccess) e = hipStreamSynchronize(s);
    if (e != hipSuccess) {
        delete c;
        return hip_fail(e, "writing the cache table");
    }

    *out = c;
    return KVQ_OK;
}

void kvq_cache_destroy(kvq_cache* c) { delete c; }

kvq_status kvq_seq_lengths(const kvq_cache* c, int32_t layer, int32_t* out) {
    g_last_error.clear();
    if (!c || !out) return fail(KVQ_ERR_ARG, "cache or out is NULL");
    if (layer < 0 || layer >= c->g.layers) return fail(KVQ_ERR_ARG, "layer %d out of range", layer);
    std::memcpy(out, &c->lens[(size_t)layer * c->g.num_seqs], sizeof(int32_t) * c->g.num_seqs);
    return KVQ_OK;
}

kvq_status kvq_get_region(const kvq_cache* c, int32_t layer, int32_t seq, kvq_region* out) {
    g_last_error.clear();
    if (!c || !out) return fail(KVQ_ERR_ARG, "cache or out is NULL");
    if (layer < 0 || layer >= c->g.layers) return fail(KVQ_ERR_ARG, "layer %d out of range", layer);
    if (seq < 0 || seq >= c->g.num_seqs) return fail(KVQ_ERR_ARG, "seq %d out of range", seq);
    const SeqEntry& e = c->entries[(size_t)layer * c->g.num_seqs + seq];
    out->k_codes = e.codes[0];
    out->v_codes = e.codes[1];
    out->k_meta = e.meta[0];
    out->v_meta = e.meta[1];
    out->k_resid = e.resid[0];
    out->v_resid = e.resid[1];
    out->k_codes_head_stride = e.codes_hs[0];
    out->v_codes_head_stride = e.codes_hs[1];
    out->k_meta_head_stride = e.meta_hs[0];
    out->v_meta_head_stride = e.meta_hs[1];
    out->k_resid_head_stride = e.resid_hs[0];
    out->v_resid_head_stride = e.resid_hs[1];
    out->bits_k = e.bits[0];
    out->bits_v = e.bits[1];
    out->capacity = e.cap;
    out->length = c->lens[(size_t)layer * c->g.num_seqs + seq];
    return KVQ_OK;
}

}  // extern "C"

namespace {

// ---- paged storage: page management on the host, mirrored to the device

int32_t* len_dev(const kvq_cache* c, int layer) {
    return (int32_t*)(c->table + c->tl.len_off) + ((size_t)c->parity[layer] * c->g.layers + layer) * c->g.num_seqs;
}

// Upload the host state of one layer: its table entries and current lengths.
kvq_status upload_layer(kvq_cache* c, int layer, hipStream_t s) {
    const int S = c->g.num_seqs;
    hipError_t e = hipMemcpyAsync(c->table + (size_t)layer * S * sizeof(SeqEntry), &c->entries[(size_t)layer * S],
                                  (size_t)S * sizeof(SeqEntry), hipMemcpyHostToDevice, s);
    if (e == hipSuccess)
        e = hipMemcpyAsync(len_dev(c, layer), &c->lens[(size_t)layer * S], (size_t)S * sizeof(int32_t),
                           hipMemcpyHostToDevice, s);
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "uploading the cache table");
}

// Upload changed page-list entries (indices into the host copy): a scatter
// kernel carrying the pairs in its arguments when they are few, else copies of
// the runs that cover them.
kvq_status upload_pages(kvq_cache* c, std::vector<uint32_t>& idx, hipStream_t s) {
    if (idx.empty()) return KVQ_OK;
    std::sort(idx.begin(), idx.end());
    idx.erase(std::unique(idx.begin(), idx.end()), idx.end());
    uint32_t* dev = (uint32_t*)(c->table + c->tl.pt_off);
    hipError_t e = hipSuccess;
    if (idx.size() <= (size_t)kvq::kPageUpdateMax) {
        kvq::PageUpdates u;
        u.count = (int32_t)idx.size();
        for (size_t i = 0; i < idx.size(); ++i) {
            u.index[i] = idx[i];
            u.value[i] = c->pt[idx[i]];
        }
        e = kvq::launch_page_updates(dev, u, s);
    } else {
        size_t a = 0;
        for (size_t i = 1; i <= idx.size() && e == hipSuccess; ++i) {
            if (i < idx.size() && idx[i] <= idx[i - 1] + 64) continue;
            const size_t n = idx[i - 1] + 1 - idx[a];
            e = hipMemcpyAsync(dev + idx[a], c->pt.data() + idx[a], n * sizeof(uint32_t), hipMemcpyHostToDevice, s);
            a = i;
        }
    }
    return e == hipSuccess ? KVQ_OK : hip_fail(e, "uploading page lists");
}

void release_page(kvq_cache* c, uint32_t p) {
    if (p == kvq::kNoPage) return;
    if (--c->refs[p] == 0) c->free_pages.push_back(p);
}

uint32_t take_page(kvq_cache* c) {
    const uint32_t p = c->free_pages.back();
    c->free_pages.pop_back();
    c->refs[p] = 1;
    return p;
}

// Map every page an append writes into (tokens [len, len + n_new[s]) of each
// sequence, in layers [layer, layer + n_layers)) that has no page yet, after
// checking that the pool has enough free pages.
kvq_status map_append_pages(kvq_cache* c, int32_t layer, int32_t n_layers, const int32_t* n_new, hipStream_t s) {
    if (!c->paged) return KVQ_OK;
    const int S = c->g.num_seqs;
    size_t need = 0;
    for (int l = layer; l < layer + n_layers; ++l)
        for (int q = 0; q < S; ++q) {
            if (!n_new[q]) continue;
            const SeqEntry& e = c->entries[(size_t)l * S + q];
            const int len = c->lens[(size_t)l * S + q];
            for (int i = len >> e.page_shift; i <= (len + n_new[q] - 1) >> e.page_shift; ++i)
                need += c->pt[(size_t)e.page_list + i] == kvq::kNoPage;
        }
    if (need > c->free_pages.size())
        return fail(KVQ_ERR_CAPACITY, "page pool exhausted: the append needs %zu new pages, %zu are free", need,
                    c->free_pages.size());
    std::vector<uint32_t> changed;
    for (int l = layer; l < layer + n_layers; ++l)
        for (int q = 0; q < S; ++q) {
            if (!n_new[q]) continue;
            const SeqEntry& e = c->entries[(size_t)l * S + q];
            const int len = c->lens[(size_t)l * S + q];
            for (int i = len >> e.page_shift; i <= (len + n_new[q] - 1) >> e.page_shift; ++i) {
                uint32_t& slot = c->pt[(size_t)e.page_list + i];
                if (slot != kvq::kNoPage) continue;
                slot = take_page(c);
                changed.push_back(e.page_list + i);
            }
        }
    return upload_pages(c, changed, s);
}

// Quantize-append of the same per-sequence counts into layers [layer, layer +
// n_layers) in one launch (1 <= n_layers <= 64, checked by the callers).
// k_new, v_new: [n_layers][sum n_new][kv_heads][head_dim].
// Validate an append and build its launch arguments (uploading non-uniform
// counts); *empty when no sequence gains a token (nothing to launch).
kvq_status prepare_append(kvq_cache* c, int32_t layer, int32_t n_layers, const void* k_new, const void* v_new,
                          const int32_t* n_new, void* stream, kvq::TensorArgs (&ta)[2], int (&gx)[2], bool* empty,
                          int* max_new) {
    const kvq_geometry& g = c->g;
    *empty = false;
    const int S = g.num_seqs;
    long total = 0;
    int max_n = 0;
    bool uniform = true;
    for (int s = 0; s < S; ++s) {
        if (n_new[s] < 0) return fail(KVQ_ERR_ARG, "n_new[%d] = %d is negative", s, n_new[s]);
        for (int l = layer; l < layer + n_layers; ++l) {
            const int len = c->lens[(size_t)l * S + s];
            if ((long)len + n_new[s] > c->cap[s])
                return fail(KVQ_ERR_CAPACITY, "layer %d sequence %d: length %d + %d exceeds capacity %d", l, s, len,
                            n_new[s], c->cap[s]);
        }
        total += n_new[s];
        max_n = std::max(max_n, n_new[s]);
        uniform = uniform && n_new[s] == n_new[0];
    }
    if (total == 0) {
        *empty = true;
        return KVQ_OK;
    }
    if (!k_new || !v_new) return fail(KVQ_ERR_ARG, "k_new and v_new must be non-NULL when tokens are appended");
    if (!aligned(k_new, 16) || !aligned(v_new, 16)) return fail(KVQ_ERR_ALIGN, "k_new and v_new must be 16-byte aligned");
    if (total > (1L << 30)) return fail(KVQ_ERR_ARG, "too many tokens in one append");

    hipStream_t hs = (hipStream_t)stream;
    const int32_t* d_n = nullptr;
    const int32_t* d_start = nullptr;
    int32_t* args_dev = (int32_t*)(c->table + c->tl.args_off);
    if (!uniform) {
        // the counts and row offsets travel in the arguments of a small scatter
        // kernel (a host-to-device copy from pageable memory would make the host
        // wait for the stream)
        kvq::PageUpdates u;
        u.count = 0;
        int32_t acc = 0;
        hipError_t e = hipSuccess;
        for (int s = 0; s < S && e == hipSuccess; ++s) {
            const int32_t vals[2] = {n_new[s], acc};
            acc += n_new[s];
            for (int k = 0; k < 2; ++k) {
                u.index[u.count] = (uint32_t)(k * S + s);
                u.value[u.count] = (uint32_t)vals[k];
                if (++u.count == kvq::kPageUpdateMax) {
                    e = kvq::launch_page_updates((uint32_t*)args_dev, u, hs);
                    u.count = 0;
                }
            }
        }
        if (e == hipSuccess) e = kvq::launch_page_updates((uint32_t*)args_dev, u, hs);
        if (e != hipSuccess) return hip_fail(e, "uploading append counts");
        d_n = args_dev;
        d_start = args_dev + S;
    }
    int32_t* len_base = (int32_t*)(c->table + c->tl.len_off);
    const int p = c->parity[layer];
    const SeqEntry* entries = (const SeqEntry*)c->table + (size_t)layer * S;

    const void* srcs[2] = {k_new, v_new};
    const int groups[2] = {g.group_k, g.group_v};
    const int axes[2] = {g.axis_k, g.axis_v};
    for (int t = 0; t < 2; ++t) {
        kvq::TensorArgs& a = ta[t];
        a = kvq::TensorArgs{};
        a.src = srcs[t];
        a.codes = c->codes;
        a.meta = meta_pool(c);
        a.resid = c->resid;
        a.pages = page_lists(c);
        a.table = entries;
        a.len_in = len_base + ((size_t)p * g.layers + layer) * S;
        a.len_out = t == 0 ? len_base + ((size_t)(1 - p) * g.layers + layer) * S : nullptr;
        a.n_new = d_n;
        a.row_start = d_start;
        a.n_uniform = uniform ? n_new[0] : 0;
        a.tensor = t;
        a.num_seqs = S;
        a.kv_heads = g.kv_heads;
        a.head_dim = g.head_dim;
        a.group = groups[t];
        a.in_dtype = g.in_dtype;
        a.axis = axes[t];
        a.rows_per_block = kvq::kThreads / (g.head_dim / 32);
        a.n_layers = n_layers;
        a.layers_total = g.layers;
        a.layer0 = layer;
        a.len_base = len_base;
        for (int i = 0; i < n_layers; ++i) a.len_parity |= (uint64_t)(c->parity[layer + i] & 1) << i;
        a.src_layer_bytes = (uint64_t)total * g.kv_heads * g.head_dim * in_bytes(g.in_dtype);
        a.win_mode = win_mode(g);
        a.sinks = g.sinks;
        a.win_rows = win_rows(g);
        a.win_off = win_off(g, t);
        if (axes[t] == KVQ_AXIS_TOKEN) {
            gx[t] = std::max(1, (max_n + a.rows_per_block - 1) / a.rows_per_block);
        } else {
            gx[t] = 1;  // completed blocks per (seq, head), at most
            for (int l = layer; l < layer + n_layers; ++l)
                for (int s = 0; s < S; ++s) {
                    const int len = c->lens[(size_t)l * S + s];
                    gx[t] = std::max(gx[t], (len + n_new[s]) / groups[t] - len / groups[t]);
                }
            if (kvq::quant_wave_path(groups[t], g.head_dim, g.in_dtype))  // four blocks per workgroup
                gx[t] = (gx[t] + kvq::kQuantBlocksPerGroup - 1) / kvq::kQuantBlocksPerGroup;
        }
    }
    if ((long)gx[0] + gx[1] > INT32_MAX / 2) return fail(KVQ_ERR_ARG, "append too large for one launch");
    *max_new = max_n;
    return map_append_pages(c, layer, n_layers, n_new, hs);
}

// The launch of a prepared append: quantize (and the full-precision window copy).
hipError_t launch_append(const kvq::TensorArgs (&ta)[2], const int (&gx)[2], int max_new, hipStream_t s) {
    return kvq::launch_quant_append(ta[0], ta[1], gx[0], gx[1], max_new, s);
}

// The host side of an append that has been launched: lengths and buffer parity.
void commit_append(kvq_cache* c, int32_t layer, int32_t n_layers, const int32_t* n_new) {
    const int S = c->g.num_seqs;
    for (int l = layer; l < layer + n_layers; ++l) {
        for (int s = 0; s < S; ++s) c->lens[(size_t)l * S + s] += n_new[s];
        c->parity[l] ^= 1;
    }
}

kvq_status append_layers(kvq_cache* c, int32_t layer, int32_t n_layers, const void* k_new, const void* v_new,
                         const int32_t* n_new, void* stream) {
    kvq::TensorArgs ta[2];
    int gx[2], max_new = 0;
    bool empty;
    kvq_status st = prepare_append(c, layer, n_layers, k_new, v_new, n_new, stream, ta, gx, &empty, &max_new);
    if (st != KVQ_OK || empty) return st;
    hipError_t e = launch_append(ta, gx, max_new, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "launching the quantize kernel");
    commit_append(c, layer, n_layers, n_new);
    return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_quantize_append(kvq_cache* c, int32_t layer, const void* k_new, const void* v_new,
                               const int32_t* n_new, void* stream) {
    g_last_error.clear();
    if (!c || !n_new) return fail(KVQ_ERR_ARG, "cache or n_new is NULL");
    if (layer < 0 || layer >= c->g.layers) return fail(KVQ_ERR_ARG, "layer %d out of range", layer);
    return append_layers(c, layer, 1, k_new, v_new, n_new, stream);
}

kvq_status kvq_quantize_append_layers(kvq_cache* c, int32_t layer0, int32_t n_layers, const void* k_new,
                                      const void* v_new, const int32_t* n_new, void* stream) {
    g_last_error.clear();
    if (!c || !n_new) return fail(KVQ_ERR_ARG, "cache or n_new is NULL");
    if (n_layers < 1 || layer0 < 0 || layer0 > c->g.layers - n_layers)
        return fail(KVQ_ERR_ARG, "layers [%d, %d + %d) out of range", layer0, layer0, n_layers);
    if (n_layers > 64) return fail(KVQ_ERR_UNSUPPORTED, "%d layers in one call (at most 64)", n_layers);
    return append_layers(c, layer0, n_layers, k_new, v_new, n_new, stream);
}

kvq_status kvq_decode_kernel(const kvq_cache* c, int32_t* kernel) {
    if (!c || !kernel) return fail(KVQ_ERR_ARG, "cache or kernel is NULL");
    const int32_t route = decode_route(c);
    if (route == KVQ_DECODE_GENERIC && group_size(c) > kvq::kMaxQueryGroup)
        return fail(KVQ_ERR_UNSUPPORTED, "q_heads / kv_heads = %d exceeds %d on the generic decode kernel",
                    group_size(c), kvq::kMaxQueryGroup);
    if (c->g.rope_base > 0.0 && c->g.axis_k != KVQ_AXIS_CHANNEL)
        return fail(KVQ_ERR_UNSUPPORTED, "rotary keys need channel-axis keys in this build");
    *kernel = route;
    return KVQ_OK;
}

size_t kvq_decode_workspace_size(const kvq_cache* c) {
    if (!c) return 0;
    const kvq_geometry& g = c->g;
    const uint64_t chunks = std::max<uint64_t>(1, (c->max_cap + min_chunk(c) - 1) / min_chunk(c)) + win_splits(c);
    const uint64_t slots = (uint64_t)g.num_seqs * g.q_heads * chunks;
    return align_up(slots * 2 * 4, kvq::kAlign) + align_up(slots * g.head_dim * 4, kvq::kAlign);
}

}  // extern "C"

namespace {

// Decode attention of layers [layer, layer + n_layers) in one launch per
// kernel (1 <= n_layers <= 64, checked by the callers; the length-buffer
// parities travel as a 64-bit mask). q, out: [n_layers][S][Hq][D].
// Options of a decode call inside a decode step (kvq_decode_step).
struct StepOpts {
    const int32_t* add = nullptr;         // host [num_seqs]: tokens the step appends (lengths seen = current + add)
    bool dry_run = false;                 // validate only
    const kvq::TensorArgs* fused = nullptr;  // [2]: the append, fused into the single-query kernel
};

kvq_status decode_layers(const kvq_cache* c, int32_t layer, int32_t n_layers, const void* q, float softmax_scale,
                         float* out, void* workspace, size_t workspace_bytes, void* stream, const StepOpts& opt = {}) {
    const kvq_geometry& g = c->g;
    const bool rope = g.rope_base > 0.0;
    if (rope && g.axis_k != KVQ_AXIS_CHANNEL)
        return fail(KVQ_ERR_UNSUPPORTED, "rotary keys need channel-axis keys in this build");
    if (!(softmax_scale == softmax_scale)) return fail(KVQ_ERR_ARG, "softmax_scale is NaN");
    if (!aligned(q, in_bytes(g.in_dtype)) || !aligned(out, 4)) return fail(KVQ_ERR_ALIGN, "q or out misaligned");
    const int S = g.num_seqs;
    const int32_t* lens = &c->lens[(size_t)layer * S];
    std::vector<int32_t> step_lens;
    if (opt.add) {  // one layer: the lengths after the step's append
        step_lens.assign(lens, lens + S);
        for (int s = 0; s < S; ++s) step_lens[s] += opt.add[s];
        lens = step_lens.data();
    }
    const int max_len = *std::max_element(lens, lens + (size_t)S * n_layers);
    const int32_t route = decode_route(c);
    const bool mha = route == KVQ_DECODE_SINGLE_QUERY;
    const bool gqa = route == KVQ_DECODE_QUERY_GROUP;
    if (!mha && !gqa && group_size(c) > kvq::kMaxQueryGroup)
        return fail(KVQ_ERR_UNSUPPORTED, "q_heads / kv_heads = %d exceeds %d on the generic decode kernel",
                    group_size(c), kvq::kMaxQueryGroup);
    const int C = mha   ? choose_split_mha(c, max_len, n_layers)
                  : gqa ? choose_split_gqa(c, lens, n_layers)
                        : choose_chunk(c, max_len, n_layers);
    // the full-precision window's slots after the quantized splits (the
    // single-query kernel's last split reads those rows itself: none there)
    const int wsl = mha ? 0 : win_splits(c);
    const int max_chunks = (mha ? std::max(1, max_len / C) : std::max(1, (max_len + C - 1) / C)) + wsl;
    const uint64_t slots = (uint64_t)n_layers * S * g.q_heads * max_chunks;
    const uint64_t ml_bytes = align_up(slots * 2 * 4, kvq::kAlign);
    const uint64_t need = ml_bytes + align_up(slots * g.head_dim * 4, kvq::kAlign);
    if (!workspace || workspace_bytes < need)
        return fail(KVQ_ERR_WORKSPACE, "workspace of %zu bytes, %llu needed", workspace_bytes, (unsigned long long)need);
    if (!aligned(workspace, kvq::kAlign)) return fail(KVQ_ERR_ALIGN, "workspace must be 256-byte aligned");
    if (opt.dry_run) return KVQ_OK;
    kvq::DecodeArgs a{};
    a.q = q;
    a.out = out;
    a.ws_ml = (float*)workspace;
    a.ws_o = (float*)((uint8_t*)workspace + ml_bytes);
    a.codes = c->codes;
    a.meta = meta_pool(c);
    a.resid = c->resid;
    a.pages = page_lists(c);
    a.table = (const SeqEntry*)c->table + (size_t)layer * S;
    a.len = (const int32_t*)(c->table + c->tl.len_off) + ((size_t)c->parity[layer] * g.layers + layer) * S;
    a.qscale = softmax_scale * 1.4426950408889634f;
    a.num_seqs = S;
    a.kv_heads = g.kv_heads;
    a.q_heads = g.q_heads;
    a.head_dim = g.head_dim;
    a.group_k = g.group_k;
    a.group_v = g.group_v;
    a.axis_k = g.axis_k;
    a.axis_v = g.axis_v;
    a.in_dtype = g.in_dtype;
    a.chunk = C;
    a.max_chunks = max_chunks;
    a.counters = (int32_t*)(c->table + c->tl.ctr_off);
    a.waves_per_group = 4;
    a.n_layers = n_layers;
    a.layers_total = g.layers;
    a.layer0 = layer;
    a.len_base = (const int32_t*)(c->table + c->tl.len_off);
    for (int i = 0; i < n_layers; ++i) a.len_parity |= (uint64_t)(c->parity[layer + i] & 1) << i;
    a.log2_group_k = __builtin_ctz((unsigned)g.group_k);
    a.log2_group_v = __builtin_ctz((unsigned)g.group_v);
    a.split_floor = mha ? 1 : 0;
    a.rope_base = g.rope_base;
    if (rope) {
        a.rope_theta = (const double*)(c->table + c->tl.rope_off);
        a.rope_tab = (const float*)(c->table + c->tl.rope_off + (size_t)g.head_dim / 2 * 8);
    }
    if (win_mode(g)) {
        a.win_mode = 1;
        a.window = g.window;
        a.sinks = g.sinks;
        a.tblock = token_block(g);
        a.win_rows = win_rows(g);
        a.win_off[0] = win_off(g, 0);
        a.win_off[1] = win_off(g, 1);
        a.ws_scale = 1.0f;  // the query-group and generic kernels' partials carry no factor
        a.win_splits = wsl;
    }
    if (a.win_mode) {
        if (!mha) {  // the full-precision rows' partials (the single-query kernel reads those rows itself)
            hipError_t e = kvq::launch_decode_window(a, (hipStream_t)stream);
            if (e != hipSuccess) return hip_fail(e, "launching the window attention");
        }
    }
    if (mha) {
        if (opt.fused) {
            a.append_fused = 1;
            a.app_k = opt.fused[0];
            a.app_v = opt.fused[1];
        }
        for (const auto& pr : c->pairs) {
            a.seq_list = c->pairs.size() == 1 ? nullptr : (const int32_t*)(c->table + c->tl.pairs_off) + pr.offset;
            hipError_t e = rope ? kvq::launch_decode_mha_rope(a, pr.bk, pr.bv, pr.count, (hipStream_t)stream)
                                : kvq::launch_decode_mha(a, pr.bk, pr.bv, pr.count, (hipStream_t)stream);
            if (e != hipSuccess) return hip_fail(e, "launching decode attention");
        }
        if (max_chunks > 1) {
            if (opt.fused) {  // the merge reads the lengths the decode kernel wrote
                a.append_fused = 0;
                a.len = opt.fused[0].len_out;
            }
            a.split_floor = 1;
            hipError_t e = kvq::launch_merge(a, (hipStream_t)stream);
            if (e != hipSuccess) return hip_fail(e, "launching the split merge");
        }
        return KVQ_OK;
    }
    if (gqa) {
        if ((long)n_layers * S <= kvq::kGqaListMax) {
            // one launch over every bit pair: the active (layer, seq) entries in
            // bit-pair order, each with its splits x kv heads x query groups
            kvq::GqaList list;
            list.count = 0;
            int items = 0;
            const int nh = g.kv_heads * ((group_size(c) + 15) / 16);
            for (const auto& pr : c->pairs)
                for (int l = 0; l < n_layers; ++l)
                    for (int i = 0; i < pr.count; ++i) {
                        const int s2 = c->pair_list[pr.offset + i];
                        int tb = 0, te = lens[(size_t)l * S + s2];
                        if (win_mode(g)) {
                            const int r = te - g.window, blk = token_block(g);
                            const int q = r > 0 ? r / blk * blk : 0;
                            tb = g.sinks;
                            te = std::max(q, g.sinks);
                        }
                        const int nsplit = te > tb ? (te - tb + C - 1) / C : 0;
                        if (!nsplit) continue;
                        list.start[list.count] = items;
                        list.seq[list.count] = (uint16_t)s2;
                        list.layer[list.count] = (uint8_t)l;
                        ++list.count;
                        items += nsplit * nh;
                    }
            list.start[list.count] = items;
            if (items > 0) {
                hipError_t e = !rope                  ? kvq::launch_decode_gqa_list(a, list, items, (hipStream_t)stream)
                               : g.head_dim == 128 ? kvq::launch_decode_gqa_rope_list_d128(a, list, items, (hipStream_t)stream)
                                                   : kvq::launch_decode_gqa_rope_list_d256(a, list, items, (hipStream_t)stream);
                if (e != hipSuccess) return hip_fail(e, "launching decode attention");
            }
        } else {
            for (const auto& pr : c->pairs) {
                a.seq_list = c->pairs.size() == 1 ? nullptr : (const int32_t*)(c->table + c->tl.pairs_off) + pr.offset;
                hipError_t e =
                    !rope               ? kvq::launch_decode_gqa(a, pr.bk, pr.bv, pr.count, (hipStream_t)stream)
                    : g.head_dim == 128 ? kvq::launch_decode_gqa_rope_d128(a, pr.bk, pr.bv, pr.count, (hipStream_t)stream)
                                        : kvq::launch_decode_gqa_rope_d256(a, pr.bk, pr.bv, pr.count, (hipStream_t)stream);
                if (e != hipSuccess) return hip_fail(e, "launching decode attention");
            }
        }
        a.split_floor = 0;
        hipError_t e = kvq::launch_merge(a, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "launching the split merge");
        return KVQ_OK;
    }
    hipError_t e = kvq::launch_decode(a, (hipStream_t)stream);
    if (e == hipSuccess) e = kvq::launch_merge(a, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "launching decode attention");
    return KVQ_OK;
}

}  // namespace

extern "C" {

kvq_status kvq_decode_attention(const kvq_cache* c, int32_t layer, const void* q, float softmax_scale, float* out,
                                void* workspace, size_t workspace_bytes, void* stream) {
    g_last_error.clear();
    if (!c || !q || !out) return fail(KVQ_ERR_ARG, "cache, q or out is NULL");
    if (layer < 0 || layer >= c->g.layers) return fail(KVQ_ERR_ARG, "layer %d out of range", layer);
    return decode_layers(c, layer, 1, q, softmax_scale, out, workspace, workspace_bytes, stream);
}

kvq_status kvq_decode_step(kvq_cache* c, int32_t layer, const void* k_new, const void* v_new, const int32_t* n_new,
                           const void* q, float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                           void* stream) {
    g_last_error.clear();
    if (!c || !n_new || !q || !out) return fail(KVQ_ERR_ARG, "cache, n_new, q or out is NULL");
    const kvq_geometry& g = c->g;
    if (layer < 0 || layer >= g.layers) return fail(KVQ_ERR_ARG, "layer %d out of range", layer);
    const int S = g.num_seqs;
    for (int s = 0; s < S; ++s)
        if (n_new[s] < 0) return fail(KVQ_ERR_ARG, "n_new[%d] = %d is negative", s, n_new[s]);
    StepOpts opt;
    opt.add = n_new;
    opt.dry_run = true;
    kvq_status st = decode_layers(c, layer, 1, q, softmax_scale, out, workspace, workspace_bytes, stream, opt);
    if (st != KVQ_OK) return st;
    kvq::TensorArgs ta[2];
    int gx[2], max_new = 0;
    bool empty;
    st = prepare_append(c, layer, 1, k_new, v_new, n_new, stream, ta, gx, &empty, &max_new);
    if (st != KVQ_OK) return st;
    // Fused when the single-query kernel serves the cache and the step only
    // adds residual key rows (no key block completes) and at most one
    // workgroup's worth of value rows per sequence.
    const int32_t* lens = &c->lens[(size_t)layer * S];
    const bool rope = g.rope_base > 0.0;
    bool fuse = !empty && group_size(c) == 1 && g.axis_k == KVQ_AXIS_CHANNEL && g.axis_v == KVQ_AXIS_TOKEN &&
                kvq::mha_supported(g.head_dim);
    for (int s = 0; fuse && s < S; ++s)
        fuse = (lens[s] + n_new[s]) / g.group_k == lens[s] / g.group_k && n_new[s] <= 256 / (g.head_dim / 32);
    for (const auto& pr : c->pairs)
        fuse = fuse && (rope ? kvq::mha_rope_fused_ok(g.head_dim, pr.bk, pr.bv)
                             : kvq::mha_fused_ok(g.head_dim, pr.bk, pr.bv));
    opt.dry_run = false;
    if (fuse) {
        opt.fused = ta;
        st = decode_layers(c, layer, 1, q, softmax_scale, out, workspace, workspace_bytes, stream, opt);
        if (st != KVQ_OK) return st;
        commit_append(c, layer, 1, n_new);
        return KVQ_OK;
    }
    if (!empty) {
        hipError_t e = launch_append(ta, gx, max_new, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "launching the quantize kernel");
        commit_append(c, layer, 1, n_new);
    }
    return decode_layers(c, layer, 1, q, softmax_scale, out, workspace, workspace_bytes, stream);
}

kvq_status kvq_decode_attention_noalloc(const kvq_cache* c, int32_t layer, const void* q, float softmax_scale,
                                       float* out, void* stream) {
    g_last_error.clear();
    if (!c || !q || !out) return fail(KVQ_ERR_ARG, "cache, q or out is NULL");
    if (layer < 0 || layer >= c->g.layers) return fail(KVQ_ERR_ARG, "layer %d out of range", layer);
    void* ws = nullptr;
    hipError_t e = kvq::scratch_address(&ws);
    if (e != hipSuccess) return hip_fail(e, "taking the address of the library's scratch");
    StepOpts opt;
    opt.dry_run = true;
    kvq_status st = decode_layers(c, layer, 1, q, softmax_scale, out, ws, kvq::kScratchBytes, stream, opt);
    if (st == KVQ_ERR_WORKSPACE)
        return fail(KVQ_ERR_WORKSPACE,
                    "this call's split workspace exceeds the library's fixed scratch of %zu bytes (use "
                    "kvq_decode_attention with a workspace of kvq_decode_workspace_size bytes)",
                    (size_t)kvq::kScratchBytes);
    if (st != KVQ_OK) return st;
    return decode_layers(c, layer, 1, q, softmax_scale, out, ws, kvq::kScratchBytes, stream);
}

kvq_status kvq_decode_attention_layers(const kvq_cache* c, int32_t layer0, int32_t n_layers, const void* q,
                                       float softmax_scale, float* out, void* workspace, size_t workspace_bytes,
                                       void* stream) {
    g_last_error.clear();
    if (!c || !q || !out) return fail(KVQ_ERR_ARG, "cache, q or out is NULL");
    if (n_layers < 1 || layer0 < 0 || layer0 > c->g.layers - n_layers)
        return fail(KVQ_ERR_ARG, "layers [%d, %d + %d) out of range", layer0, layer0, n_layers);
    if (n_layers > 64) return fail(KVQ_ERR_UNSUPPORTED, "%d layers in one call (at most 64)", n_layers);
    return decode_layers(c, layer0, n_layers, q, softmax_scale, out, workspace, workspace_bytes, stream);
}

kvq_status kvq_dequantize(const kvq_cache* c, int32_t layer, int32_t seq, float* k_out, float* v_out, void* stream) {
    g_last_error.clear();
    if (!c) return fail(KVQ_ERR_ARG, "cache is NULL");
    const kvq_geometry& g = c->g;
    if (layer < 0 || layer >= g.layers) return fail(KVQ_ERR_ARG, "layer %d out of range", layer);
    if (seq < 0 || seq >= g.num_seqs) return fail(KVQ_ERR_ARG, "seq %d out of range", seq);
    if ((k_out && !aligned(k_out, 4)) || (v_out && !aligned(v_out, 4))) return fail(KVQ_ERR_ALIGN, "outputs misaligned");
    const int len = c->lens[(size_t)layer * g.num_seqs + seq];
    float* outs[2] = {k_out, v_out};
    const int groups[2] = {g.group_k, g.group_v};
    const int axes[2] = {g.axis_k, g.axis_v};
    for (int t = 0; t < 2; ++t) {
        if (!outs[t]) continue;
        kvq::DequantArgs a{};
        a.out = outs[t];
        a.codes = c->codes;
        a.meta = meta_pool(c);
        a.resid = c->resid;
        a.pages = page_lists(c);
        a.entry = c->entries[(size_t)layer * g.num_seqs + seq];
        a.tensor = t;
        a.len = len;
        a.kv_heads = g.kv_heads;
        a.head_dim = g.head_dim;
        a.group = groups[t];
        a.axis = axes[t];
        a.in_dtype = g.in_dtype;
        if (win_mode(g)) {
            a.win_mode = 1;
            a.window = g.window;
            a.sinks = g.sinks;
            a.tblock = token_block(g);
            a.win_rows = win_rows(g);
            a.win_off = win_off(g, t);
        }
        hipError_t e = kvq::launch_dequant(a, (hipStream_t)stream);
        if (e != hipSuccess) return hip_fail(e, "launching dequantize");
    }
    return KVQ_OK;
}

kvq_status kvq_gather_sequences(kvq_cache* c, int32_t layer0, int32_t n_layers, const int32_t* src, void* stream) {
    g_last_error.clear();
    if (!c || !src) return fail(KVQ_ERR_ARG, "cache or src is NULL");
    const kvq_geometry& g = c->g;
    const int S = g.num_seqs;
    if (n_layers < 1 || layer0 < 0 || layer0 > g.layers - n_layers)
        return fail(KVQ_ERR_ARG, "layers [%d, %d + %d) out of range", layer0, layer0, n_layers);
    for (int q = 0; q < S; ++q) {
        if (src[q] < 0 || src[q] >= S) return fail(KVQ_ERR_ARG, "src[%d] = %d out of range", q, src[q]);
        const int o = src[q];
        if (c->bits_k[q] != c->bits_k[o] || c->bits_v[q] != c->bits_v[o] || c->cap[q] != c->cap[o])
            return fail(KVQ_ERR_ARG, "sequences %d and %d differ in bits or capacity", q, o);
    }
    // keeper[o]: the sequence that takes o's own regions and pages (o itself
    // when it stays, else the first sequence copying it); -1: o is dropped
    std::vector<int> keeper(S, -1);
    for (int q = 0; q < S; ++q)
        if (src[q] == q) keeper[q] = q;
    for (int q = 0; q < S; ++q)
        if (keeper[src[q]] < 0) keeper[src[q]] = q;
    const int P = g.page_tokens;
    auto partial_page = [&](int len) { return P && len % P ? len / P : -1; };  // index of a page still filling
    if (c->paged) {  // enough free pages for the extra copies of incomplete pages, counting the call's releases
        std::vector<uint32_t> refs = c->refs;
        size_t freed = 0, need = 0;
        for (int l = layer0; l < layer0 + n_layers; ++l) {
            for (int q = 0; q < S; ++q) {
                const SeqEntry& eo = c->entries[(size_t)l * S + src[q]];
                const uint32_t used = pages_of(&g, c->lens[(size_t)l * S + src[q]]);
                for (uint32_t i = 0; i < used; ++i)
                    if (c->pt[(size_t)eo.page_list + i] != kvq::kNoPage) ++refs[c->pt[(size_t)eo.page_list + i]];
                if (keeper[src[q]] != q && partial_page(c->lens[(size_t)l * S + src[q]]) >= 0) ++need;
            }
            for (int q = 0; q < S; ++q) {
                const SeqEntry& e = c->entries[(size_t)l * S + q];
                for (uint32_t i = 0; i < pages_of(&g, c->cap[q]); ++i) {
                    const uint32_t p = c->pt[(size_t)e.page_list + i];
                    if (p != kvq::kNoPage && --refs[p] == 0) ++freed;
                }
            }
        }
        if (need > c->free_pages.size() + freed)
            return fail(KVQ_ERR_CAPACITY, "page pool exhausted: the gather needs %zu new pages, %zu are free", need,
                        c->free_pages.size() + freed);
    }
    hipStream_t hs = (hipStream_t)stream;
    const uint64_t H = g.kv_heads, D = g.head_dim;
    for (int l = layer0; l < layer0 + n_layers; ++l) {
        const size_t base = (size_t)l * S;
        // regions: a dropped sequence's slot goes to an extra copy of the same class
        std::vector<int32_t> new_slot(S, -1);
        std::vector<int> spare;  // dropped sequences, by class when taken
        for (int o = 0; o < S; ++o)
            if (keeper[o] < 0) spare.push_back(o);
        std::vector<int> copies;  // sequences that receive a copy
        for (int q = 0; q < S; ++q) {
            if (keeper[src[q]] == q) {
                new_slot[q] = c->slot[base + src[q]];
                continue;
            }
            for (size_t i = 0; i < spare.size(); ++i) {
                const int o = spare[i];
                if (o >= 0 && c->bits_k[o] == c->bits_k[q] && c->bits_v[o] == c->bits_v[q] && c->cap[o] == c->cap[q]) {
                    new_slot[q] = c->slot[base + o];
                    spare[i] = -1;
                    break;
                }
            }
            if (new_slot[q] < 0) return fail(KVQ_ERR_ARG, "no region of sequence %d's class is free", q);  // unreachable
            copies.push_back(q);
        }
        for (int q : copies) {
            const int o = src[q];
            const SeqEntry& from = c->slot_layout[base + c->slot[base + o]];
            const SeqEntry& to = c->slot_layout[base + new_slot[q]];
            const int len = c->lens[base + o];
            for (int t = 0; t < 2; ++t) {
                hipError_t e = hipSuccess;
                if (from.resid_hs[t])
                    e = hipMemcpyAsync(c->resid + to.resid[t], c->resid + from.resid[t], from.resid_hs[t] * H,
                                       hipMemcpyDeviceToDevice, hs);
                if (!c->paged && e == hipSuccess) {
                    // the first len rows of codes and their metadata, every head
                    const bool ch = (t == 0 ? g.axis_k : g.axis_v) == KVQ_AXIS_CHANNEL;
                    const uint64_t G = t == 0 ? g.group_k : g.group_v, B = from.bits[t];
                    const uint64_t rows = ch ? len / G * G : len;
                    const uint64_t cb = rows * D * B / 8, mb = (ch ? len / G * D : (uint64_t)len * (D / G)) * 4;
                    if (cb)
                        e = hipMemcpy2DAsync(c->codes + to.codes[t], to.codes_hs[t], c->codes + from.codes[t],
                                             from.codes_hs[t], cb, H, hipMemcpyDeviceToDevice, hs);
                    if (mb && e == hipSuccess)
                        e = hipMemcpy2DAsync(c->meta + to.meta[t], to.meta_hs[t], c->meta + from.meta[t],
                                             from.meta_hs[t], mb, H, hipMemcpyDeviceToDevice, hs);
                }
                if (e != hipSuccess) return hip_fail(e, "copying a sequence");
            }
        }
        std::vector<uint32_t> changed;
        if (c->paged) {
            // new lists: the source's pages up to its length, shared; an extra
            // copy of a page still filling gets a page of its own
            std::vector<std::vector<uint32_t>> nl(S);
            for (int q = 0; q < S; ++q) {
                const SeqEntry& eo = c->entries[base + src[q]];
                const uint32_t n = pages_of(&g, c->cap[q]), used = pages_of(&g, c->lens[base + src[q]]);
                nl[q].assign(n, kvq::kNoPage);
                for (uint32_t i = 0; i < used; ++i) {
                    nl[q][i] = c->pt[(size_t)eo.page_list + i];
                    if (nl[q][i] != kvq::kNoPage) ++c->refs[nl[q][i]];
                }
            }
            for (int q = 0; q < S; ++q) {
                const SeqEntry& e = c->entries[base + q];
                for (uint32_t i = 0; i < pages_of(&g, c->cap[q]); ++i) release_page(c, c->pt[(size_t)e.page_list + i]);
            }
            for (int q : copies) {
                const int i = partial_page(c->lens[base + src[q]]);
                if (i < 0 || nl[q][i] == kvq::kNoPage) continue;
                const uint32_t p = nl[q][i], fresh = take_page(c);
                --c->refs[p];  // still held by the keeper
                nl[q][i] = fresh;
                hipError_t e = hipMemcpyAsync(c->codes + (uint64_t)fresh * c->page_bytes,
                                              c->codes + (uint64_t)p * c->page_bytes, c->page_bytes,
                                              hipMemcpyDeviceToDevice, hs);
                if (e != hipSuccess) return hip_fail(e, "copying a page");
            }
            for (int q = 0; q < S; ++q) {
                const SeqEntry& e = c->entries[base + q];
                for (uint32_t i = 0; i < nl[q].size(); ++i) {
                    uint32_t& slot = c->pt[(size_t)e.page_list + i];
                    if (slot != nl[q][i]) {
                        slot = nl[q][i];
                        changed.push_back(e.page_list + i);
                    }
                }
            }
        }
        // entries and lengths
        std::vector<SeqEntry> ne(S);
        std::vector<int32_t> nlen(S);
        for (int q = 0; q < S; ++q) {
            ne[q] = c->slot_layout[base + new_slot[q]];
            ne[q].page_list = c->entries[base + q].page_list;
            ne[q].ring = c->entries[base + src[q]].ring;
            nlen[q] = c->lens[base + src[q]];
        }
        for (int q = 0; q < S; ++q) {
            c->entries[base + q] = ne[q];
            c->slot[base + q] = new_slot[q];
            c->lens[base + q] = nlen[q];
        }
        kvq_status st = upload_pages(c, changed, hs);
        if (st == KVQ_OK) st = upload_layer(c, l, hs);
        if (st != KVQ_OK) return st;
    }
    return KVQ_OK;
}

kvq_status kvq_evict_tokens(kvq_cache* c, int32_t layer0, int32_t n_layers, int32_t seq, int32_t first, int32_t count,
                            void* stream) {
    g_last_error.clear();
    if (!c) return fail(KVQ_ERR_ARG, "cache is NULL");
    const kvq_geometry& g = c->g;
    const int S = g.num_seqs;
    if (n_layers < 1 || layer0 < 0 || layer0 > g.layers - n_layers)
        return fail(KVQ_ERR_ARG, "layers [%d, %d + %d) out of range", layer0, layer0, n_layers);
    if (seq < 0 || seq >= S) return fail(KVQ_ERR_ARG, "seq %d out of range", seq);
    if (!c->paged) return fail(KVQ_ERR_UNSUPPORTED, "eviction needs paged storage");
    if (first < 0 || count < 0) return fail(KVQ_ERR_ARG, "first (%d) and count (%d) must be >= 0", first, count);
    if (count == 0) return KVQ_OK;
    const int P = g.page_tokens;
    if (first % P || count % P) return fail(KVQ_ERR_ARG, "first and count must be multiples of page_tokens (%d)", P);
    if (first < g.sinks) return fail(KVQ_ERR_ARG, "the sinks [0, %d) cannot be evicted", g.sinks);
    for (int l = layer0; l < layer0 + n_layers; ++l) {
        const int len = c->lens[(size_t)l * S + seq];
        if ((long)first + count > (long)len / P * P)
            return fail(KVQ_ERR_ARG, "layer %d: tokens [%d, %d) are not whole pages below length %d", l, first,
                        first + count, len);
        if (win_mode(g) && (long)first + count > (long)len - win_rows(g))
            return fail(KVQ_ERR_ARG, "layer %d: tokens [%d, %d) reach the last window + block = %d tokens", l, first,
                        first + count, win_rows(g));
    }
    hipStream_t hs = (hipStream_t)stream;
    for (int l = layer0; l < layer0 + n_layers; ++l) {
        const size_t i = (size_t)l * S + seq;
        SeqEntry& e = c->entries[i];
        uint32_t* list = &c->pt[e.page_list];
        const uint32_t n = pages_of(&g, c->cap[seq]), i0 = first / P, k = count / P;
        for (uint32_t j = i0; j < i0 + k; ++j) release_page(c, list[j]);
        for (uint32_t j = i0; j < n; ++j) list[j] = j + k < n ? list[j + k] : kvq::kNoPage;
        std::vector<uint32_t> changed;
        for (uint32_t j = i0; j < n; ++j) changed.push_back(e.page_list + j);
        c->lens[i] -= count;
        if (win_mode(g)) e.ring = (int32_t)(((long)e.ring + count) % win_rows(g));
        kvq_status st = upload_pages(c, changed, hs);
        if (st == KVQ_OK) st = upload_layer(c, l, hs);
        if (st != KVQ_OK) return st;
    }
    return KVQ_OK;
}

kvq_status kvq_reset_sequence(kvq_cache* c, int32_t layer0, int32_t n_layers, int32_t seq, void* stream) {
    g_last_error.clear();
    if (!c) return fail(KVQ_ERR_ARG, "cache is NULL");
    const kvq_geometry& g = c->g;
    const int S = g.num_seqs;
    if (n_layers < 1 || layer0 < 0 || layer0 > g.layers - n_layers)
        return fail(KVQ_ERR_ARG, "layers [%d, %d + %d) out of range", layer0, layer0, n_layers);
    if (seq < 0 || seq >= S) return fail(KVQ_ERR_ARG, "seq %d out of range", seq);
    hipStream_t hs = (hipStream_t)stream;
    for (int l = layer0; l < layer0 + n_layers; ++l) {
        const size_t i = (size_t)l * S + seq;
        SeqEntry& e = c->entries[i];
        std::vector<uint32_t> changed;
        if (c->paged) {
            for (uint32_t j = 0; j < pages_of(&g, c->cap[seq]); ++j) {
                uint32_t& p = c->pt[(size_t)e.page_list + j];
                if (p == kvq::kNoPage) continue;
                release_page(c, p);
                p = kvq::kNoPage;
                changed.push_back(e.page_list + j);
            }
        }
        c->lens[i] = 0;
        e.ring = 0;
        kvq_status st = upload_pages(c, changed, hs);
        if (st == KVQ_OK) st = upload_layer(c, l, hs);
        if (st != KVQ_OK) return st;
    }
    return KVQ_OK;
}

kvq_status kvq_page_list(const kvq_cache* c, int32_t layer, int32_t seq, uint32_t* out, int32_t max_out,
                         int32_t* n_pages, int64_t* free_pages) {
    g_last_error.clear();
    if (!c || (!out && max_out > 0) || !n_pages) return fail(KVQ_ERR_ARG, "cache, out or n_pages is NULL");
    if (layer < 0 || layer >= c->g.layers) return fail(KVQ_ERR_ARG, "layer %d out of range", layer);
    if (seq < 0 || seq >= c->g.num_seqs) return fail(KVQ_ERR_ARG, "seq %d out of range", seq);
    if (!c->paged) return fail(KVQ_ERR_UNSUPPORTED, "the cache has contiguous storage");
    const SeqEntry& e = c->entries[(size_t)layer * c->g.num_seqs + seq];
    const int32_t n = (int32_t)pages_of(&c->g, c->cap[seq]);
    *n_pages = n;
    for (int32_t i = 0; i < std::min(n, max_out); ++i) out[i] = c->pt[(size_t)e.page_list + i];
    if (free_pages) *free_pages = (int64_t)c->free_pages.size();
    return KVQ_OK;
}

kvq_status kvq_copy_sequence(kvq_cache* dst, int32_t dst_seq, const kvq_cache* src, int32_t src_seq, int32_t layer0,
                             int32_t n_layers, void* stream) {
    g_last_error.clear();
    if (!dst || !src) return fail(KVQ_ERR_ARG, "cache is NULL");
    const kvq_geometry &gd = dst->g, &gs = src->g;
    const bool same = gd.layers == gs.layers && gd.num_seqs == gs.num_seqs && gd.kv_heads == gs.kv_heads &&
                      gd.q_heads == gs.q_heads && gd.head_dim == gs.head_dim && gd.group_k == gs.group_k &&
                      gd.group_v == gs.group_v && gd.axis_k == gs.axis_k && gd.axis_v == gs.axis_v &&
                      gd.in_dtype == gs.in_dtype && gd.meta_dtype == gs.meta_dtype && gd.window == gs.window &&
                      gd.sinks == gs.sinks && gd.rope_base == gs.rope_base && gd.page_tokens == gs.page_tokens &&
                      gd.num_pages == gs.num_pages;
    if (!same) return fail(KVQ_ERR_ARG, "the caches' geometries differ");
    if (dst_seq < 0 || dst_seq >= gd.num_seqs || src_seq < 0 || src_seq >= gs.num_seqs)
        return fail(KVQ_ERR_ARG, "sequence index out of range");
    if (dst == src && dst_seq == src_seq) return fail(KVQ_ERR_ARG, "a sequence copied onto itself");
    if (n_layers < 1 || layer0 < 0 || layer0 > gd.layers - n_layers)
        return fail(KVQ_ERR_ARG, "layers [%d, %d + %d) out of range", layer0, layer0, n_layers);
    if (dst->bits_k[dst_seq] != src->bits_k[src_seq] || dst->bits_v[dst_seq] != src->bits_v[src_seq] ||
        dst->cap[dst_seq] != src->cap[src_seq])
        return fail(KVQ_ERR_ARG, "the sequences' bits or capacities differ");
    if (dst->paged) {  // one cache: a gather that forks src_seq onto dst_seq
        if (dst != src) return fail(KVQ_ERR_UNSUPPORTED, "paged storage copies sequences within one cache only");
        std::vector<int32_t> map(gd.num_seqs);
        for (int q = 0; q < gd.num_seqs; ++q) map[q] = q;
        map[dst_seq] = src_seq;
        return kvq_gather_sequences(dst, layer0, n_layers, map.data(), stream);
    }
    hipStream_t hs = (hipStream_t)stream;
    const int S = gd.num_seqs;
    for (int l = layer0; l < layer0 + n_layers; ++l) {
        const SeqEntry& ed = dst->entries[(size_t)l * S + dst_seq];
        const SeqEntry& es = src->entries[(size_t)l * S + src_seq];
        for (int t = 0; t < 2; ++t) {
            // a tensor's heads are contiguous, with equal strides for equal bits and capacity
            const struct { uint8_t *d; const uint8_t* s; uint64_t n; } parts[3] = {
                {dst->codes + ed.codes[t], src->codes + es.codes[t], es.codes_hs[t] * gd.kv_heads},
                {dst->meta + ed.meta[t], src->meta + es.meta[t], es.meta_hs[t] * gd.kv_heads},
                {dst->resid + ed.resid[t], src->resid + es.resid[t], es.resid_hs[t] * gd.kv_heads}};
            for (const auto& p : parts) {
                if (p.n == 0) continue;
                hipError_t e = hipMemcpyAsync(p.d, p.s, p.n, hipMemcpyDeviceToDevice, hs);
                if (e != hipSuccess) return hip_fail(e, "copying a sequence");
            }
        }
        // the length, in the destination layer's current length buffer
        int32_t* len_dev = (int32_t*)(dst->table + dst->tl.len_off) + ((size_t)dst->parity[l] * gd.layers + l) * S;
        const int32_t* len_src = (const int32_t*)(src->table + src->tl.len_off) +
                                 ((size_t)src->parity[l] * gs.layers + l) * S;
        hipError_t e = hipMemcpyAsync(len_dev + dst_seq, len_src + src_seq, sizeof(int32_t), hipMemcpyDeviceToDevice, hs);
        if (e != hipSuccess) return hip_fail(e, "copying a sequence length");
        dst->lens[(size_t)l * S + dst_seq] = src->lens[(size_t)l * S + src_seq];
    }
    return KVQ_OK;
}

kvq_status kvq_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, void* stream) {
    g_last_error.clear();
    if (!buf || !sink) return fail(KVQ_ERR_ARG, "buffer or sink is NULL");
    if (bytes % 16 != 0) return fail(KVQ_ERR_ARG, "bytes (%llu) is not a multiple of 16", (unsigned long long)bytes);
    if (!aligned(buf, 16) || !aligned(sink, 4)) return fail(KVQ_ERR_ALIGN, "buffer not 16-byte or sink not 4-byte aligned");
    if (bytes == 0) return KVQ_OK;
    hipError_t e = kvq::launch_read_probe(buf, bytes, sink, (hipStream_t)stream);
    if (e != hipSuccess) return hip_fail(e, "launching the read probe");
    return KVQ_OK;
}

}  // extern "C"
