"""Paged storage on the GPU against the CPU oracle ([N] "State quantized cache
harus tetap selaras dengan posisi": positions are remapped to physical slots
by paging, beam operations, prefix reuse and eviction, and each page carries
the steps and zeros of the codes it holds).

The oracle knows nothing of pages: a sequence is its token history. Each test
keeps the histories in Python, applies the same forks, reorders and evictions
to them, and checks the cache against the oracle's encoding of the resulting
histories: stored bytes (read through the page lists) and kvq_dequantize bit
for bit, attention within 2e-3 of the fp64 oracle. Appends are interleaved
across sequences in uneven chunks, so physical pages are assigned out of
logical order."""

import sys

import numpy as np
import pytest
import torch

from bit_kv_cache_groupwise_amd import workloads as W
from oracle import kvq_oracle as o
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

NO_PAGE = 0xFFFFFFFF


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


class Hist:
    """Per-sequence token histories of one layer ([T][Hkv][D] float32, values
    exact in the input dtype)."""

    def __init__(self, w):
        self.w = w
        self.k = [np.zeros((0, w.kv_heads, w.head_dim), np.float32) for _ in range(w.num_seqs)]
        self.v = [x.copy() for x in self.k]
        self.draws = 0

    def append(self, cache, layer, counts, step=None):
        """Draw sum(counts) new rows, append them through the cache (kvq_decode_step
        when step = (q, scale)), and extend the histories."""
        self.draws += 1
        k, v = W.draw_kv(self.w, layer, counts, stream=100 + self.draws)
        off = W.seq_offsets(counts)
        for s in range(self.w.num_seqs):
            self.k[s] = np.concatenate([self.k[s], k[off[s]:off[s + 1]].float().numpy()])
            self.v[s] = np.concatenate([self.v[s], v[off[s]:off[s + 1]].float().numpy()])
        if step is None:
            cache.append(layer, k.cuda(), v.cuda(), counts)
            return None
        q, scale = step
        return cache.step(layer, k.cuda(), v.cuda(), counts, q, scale)

    def gather(self, src):
        self.k = [self.k[i].copy() for i in src]
        self.v = [self.v[i].copy() for i in src]

    def evict(self, s, first, count):
        keep = np.r_[0:first, first + count:len(self.k[s])]
        self.k[s], self.v[s] = self.k[s][keep], self.v[s][keep]


def scramble_pool(cache, w, layer):
    """Fill every sequence with throw-away tokens, then empty it again: the pool
    hands out pages last-freed-first, so the pages taken afterwards come in
    descending physical order and hold stale codes."""
    P = cache.geom.page_tokens
    counts = [min(c, 3 * P) for c in cache.capacity]
    k, v = W.draw_kv(w, layer, counts, stream=99)
    cache.append(layer, k.cuda(), v.cuda(), counts)
    for s in range(w.num_seqs):
        cache.reset(s, layer, 1)


def prefill(cache, hist, layer, lengths, chunks=(37, 64, 5, 100)):
    """Append the histories' first tokens in chunks that alternate between the
    sequences (after scramble_pool with paged storage), so that pages are taken
    from the pool out of logical order."""
    if cache.geom.page_tokens:
        scramble_pool(cache, hist.w, layer)
    done = [0] * len(lengths)
    i = 0
    while any(d < L for d, L in zip(done, lengths)):
        c = chunks[i % len(chunks)]
        take = [min(c, L - d) if (s + i) % 2 == 0 or c < 50 else 0 for s, (d, L) in enumerate(zip(done, lengths))]
        if not any(take):
            take = [min(c, L - d) for d, L in zip(done, lengths)]
        hist.append(cache, layer, take)
        done = [d + t for d, t in zip(done, take)]
        i += 1


def check(cache, w, layer, hist, q, out, *, window=0, sinks=0, rope=0.0, name=""):
    """Stored bytes, dequantized rows and the attention rows of every sequence
    against the oracle's encoding of its history."""
    R = w.q_heads // w.kv_heads
    worst = 0.0
    torch.cuda.synchronize()
    lens = cache.lengths(layer)
    for s in range(w.num_seqs):
        k, v = hist.k[s], hist.v[s]
        assert lens[s] == len(k), (name, s, lens[s], len(k))
        encs = []
        for h in range(w.kv_heads):
            H.assert_head_bytes(cache, w, layer, s, h, k, v)
            encs.append(H.encode_window(w, k, v, s, h, window, sinks) if (window or sinks) else H.encode(w, k, v, s, h))
        kd, vd = cache.dequantize(layer, s)
        torch.cuda.synchronize()
        for h in range(w.kv_heads):
            np.testing.assert_array_equal(kd[h].cpu().numpy(), encs[h]["k_hat"].astype(np.float32),
                                          err_msg=f"{name} k s{s} h{h}")
            np.testing.assert_array_equal(vd[h].cpu().numpy(), encs[h]["v_hat"].astype(np.float32),
                                          err_msg=f"{name} v s{s} h{h}")
        qs = q[s].double().cpu().numpy()
        for h in range(w.kv_heads):
            if rope:
                ref = o.attend_rope(qs[h * R:(h + 1) * R], encs[h]["k_hat"], encs[h]["v_hat"], w.softmax_scale, rope)
            else:
                ref = o.attend(qs[h * R:(h + 1) * R], encs[h]["k_hat"], encs[h]["v_hat"], w.softmax_scale)
            err = H.row_rel_err(out[s, h * R:(h + 1) * R], ref)
            worst = max(worst, float(err.max()))
            assert np.all(err <= H.ATTN_TOL), (name, s, h, float(err.max()))
    return worst


def shuffled(cache, w, layer):
    """Whether some sequence's pages are not in ascending physical order."""
    for s in range(w.num_seqs):
        pl = [p for p in cache.page_list(layer, s)[0] if p != NO_PAGE]
        if pl != sorted(pl):
            return True
    return False


# (workload, page tokens, window, sinks, rotary base): each decode kernel
CASES = {
    # single-query kernel (fused decode step), head_dim 128, 2-bit
    "llama": (W.llama2_7b().scaled(num_seqs=3, kv_heads=2, q_heads=2, lengths=(700, 130, 1), bits=((2, 2),) * 3),
              64, 0, 0, 0.0),
    # single-query kernel, head_dim 64, K6/V4, 64-token key blocks
    "gpt2": (W.gpt2_small().scaled(num_seqs=3, layers=1, kv_heads=2, q_heads=2, lengths=(1024, 300, 64),
                                   bits=((6, 4),) * 3), 128, 0, 0, 0.0),
    # query-group kernel over every bit pair, one launch
    "mixed": (W.mixed_batch().scaled(num_seqs=10, lengths=(0, 1, 31, 64, 65, 100, 512, 1000, 1500, 2047),
                                     bits=tuple(W.BIT_PAIRS_MIXED[i % 5] for i in range(10))), 64, 0, 0, 0.0),
    # query-group kernel, head_dim 256, bf16, K4/V8, large pages
    "gqa256": (W.long_gqa().scaled(lengths=(3000,)), 512, 0, 0, 0.0),
    # generic split kernel: per-token keys
    "ktoken": (W.gpt2_small().scaled(num_seqs=2, layers=1, kv_heads=2, q_heads=2, lengths=(300, 64),
                                     bits=((6, 4),) * 2, axis_k=o.AXIS_TOKEN), 64, 0, 0, 0.0),
    # generic split kernel: rotary keys
    "rope": (W.llama2_7b().scaled(num_seqs=2, kv_heads=2, q_heads=2, lengths=(900, 70), bits=((3, 3),) * 2),
             64, 0, 0, 10000.0),
    # full-precision window and sinks, single-query and query-group kernels
    "llama_window": (W.llama2_7b().scaled(num_seqs=2, kv_heads=2, q_heads=2, lengths=(1000, 90),
                                          bits=((2, 2),) * 2), 64, 100, 64, 0.0),
    "mixed_window": (W.mixed_batch().scaled(num_seqs=5, lengths=(40, 300, 1000, 129, 2000),
                                            bits=tuple(W.BIT_PAIRS_MIXED)), 128, 64, 128, 0.0),
}


@pytest.mark.parametrize("name", list(CASES))
def test_paged_parity(name):
    w, P, window, sinks, rope = CASES[name]
    _note(f"[paged] case={name} P={P} lens={w.lengths}")
    cache = H.make_cache(w, extra=16, page_tokens=P, window=window, sinks=sinks, rope_base=rope)
    hist = Hist(w)
    prefill(cache, hist, 0, w.lengths)
    if sum(L >= 2 * P for L in w.lengths) >= 2:
        assert shuffled(cache, w, 0), "the page lists came out in physical order: the test would not see a mix-up"
    q = W.draw_q(w, 0).cuda()
    out = hist.append(cache, 0, [w.new_tokens] * w.num_seqs, step=(q, w.softmax_scale)).cpu().numpy()
    worst = check(cache, w, 0, hist, q, out, window=window, sinks=sinks, rope=rope, name=name)
    _note(f"[paged] case={name} worst row rel err {worst:.3e}")
    cache.close()


@pytest.mark.parametrize("name", ["mixed", "llama"])
def test_paged_equals_contiguous(name):
    """The same appends into a paged and a contiguous cache: equal dequantized
    rows, and with the query-group kernel (same splits) equal attention bit for bit."""
    w, P, _, _, _ = CASES[name]
    ca = H.make_cache(w, extra=16, page_tokens=P)
    cb = H.make_cache(w, extra=16)
    ha, hb = Hist(w), Hist(w)
    prefill(ca, ha, 0, w.lengths)
    prefill(cb, hb, 0, w.lengths)
    q = W.draw_q(w, 0).cuda()
    oa = ca.decode(0, q, w.softmax_scale)
    ob = cb.decode(0, q, w.softmax_scale)
    torch.cuda.synchronize()
    if w.q_heads > w.kv_heads:
        assert torch.equal(oa, ob)
    else:
        assert np.all(H.row_rel_err(oa.cpu().numpy(), ob.cpu().numpy()) <= 1e-5)
    for s in range(w.num_seqs):
        ka, va = ca.dequantize(0, s)
        kb, vb = cb.dequantize(0, s)
        assert torch.equal(ka, kb) and torch.equal(va, vb)


@pytest.mark.parametrize("name,P", [("llama", 64), ("mixed", 128), ("gqa256", 256)])
def test_forked_beams(name, P):
    """One prompt forked into every sequence (prefix sharing), then each beam
    decodes its own tokens: the whole pages of the prompt stay shared, the page
    holding the prompt's last tokens is copied once per extra beam."""
    w = CASES[name][0]
    S = 4
    pair = w.bits[-1]
    w = w.scaled(num_seqs=S, lengths=(3 * P + 8,) + (0,) * (S - 1), bits=(pair,) * S)
    steps = 6
    cache = H.make_cache(w, capacity=[3 * P + 8 + steps * w.new_tokens + 16] * S, page_tokens=P)
    hist = Hist(w)
    prefill(cache, hist, 0, w.lengths)
    free0 = cache.page_list(0, 0)[1]
    cache.gather([0] * S)
    hist.gather([0] * S)
    lists = [cache.page_list(0, s)[0] for s in range(S)]
    for s in range(1, S):
        assert lists[s][:3] == lists[0][:3], "whole pages are shared"
        assert lists[s][3] not in (lists[0][3], NO_PAGE), "the page still filling is a copy"
    assert cache.page_list(0, 0)[1] == free0 - (S - 1)
    for st in range(steps):
        q = W.draw_q(w, 0, step=st).cuda()
        out = hist.append(cache, 0, [w.new_tokens] * S, step=(q, w.softmax_scale)).cpu().numpy()
    worst = check(cache, w, 0, hist, q, out, name=f"fork-{name}")
    _note(f"[paged fork] case={name} worst row rel err {worst:.3e}")
    # the beams' own tokens went to pages of their own: the prompt's pages are unchanged
    assert all(cache.page_list(0, s)[0][:3] == lists[0][:3] for s in range(S))
    cache.close()


@pytest.mark.parametrize("paged", [True, False], ids=["paged", "contiguous"])
@pytest.mark.parametrize("name", ["llama", "mixed_window"])
def test_beam_reorder(name, paged):
    """Beam search: after some steps the surviving beams replace the dropped
    ones (a gather with repeats); decoding continues from the reordered caches."""
    w, P, window, sinks, _ = CASES[name]
    S = 4
    pair = w.bits[-1]
    w = w.scaled(num_seqs=S, lengths=(300, 200, 450, 129), bits=(pair,) * S)
    cap = [700] * S
    cache = H.make_cache(w, capacity=cap, page_tokens=P if paged else 0, window=window, sinks=sinks)
    hist = Hist(w)
    prefill(cache, hist, 0, w.lengths)
    for src in ([2, 0, 2, 1], [1, 1, 3, 3], [3, 2, 1, 0]):
        cache.gather(src)
        hist.gather(src)
        for st in range(3):
            q = W.draw_q(w, 0, step=st).cuda()
            out = hist.append(cache, 0, [w.new_tokens] * S, step=(q, w.softmax_scale)).cpu().numpy()
        worst = check(cache, w, 0, hist, q, out, window=window, sinks=sinks, name=f"reorder-{name}-{src}")
        _note(f"[paged reorder] case={name} paged={paged} src={src} worst {worst:.3e}")
    if paged:  # every page is referred to by some sequence or free
        free = cache.page_list(0, 0)[1]
        used = set()
        for s in range(S):
            used |= {p for p in cache.page_list(0, s)[0] if p != NO_PAGE}
        assert len(used) + free == cache.sizes.num_pages
    cache.close()


@pytest.mark.parametrize("name", ["llama", "mixed", "rope", "llama_window", "mixed_window"])
def test_evict_pages(name):
    """Evicting whole pages from the middle of a sequence: the cache then holds
    the history without those tokens (later tokens move down, rotary keys are
    rotated to their new positions, the window rows stay valid), and decoding
    and appending continue."""
    w, P, window, sinks, rope = CASES[name]
    w = w.scaled(lengths=tuple(max(L, 2 * P + sinks + window + 200) if i % 2 == 0 else L
                               for i, L in enumerate(w.lengths)))
    cache = H.make_cache(w, extra=64, page_tokens=P, window=window, sinks=sinks, rope_base=rope)
    hist = Hist(w)
    prefill(cache, hist, 0, w.lengths)
    free0 = cache.page_list(0, 0)[1]
    evicted = 0
    for s in range(0, w.num_seqs, 2):
        first = max(sinks, P)
        count = P * ((w.lengths[s] - window - 64 - first) // P // 2)
        if count <= 0:
            continue
        cache.evict(s, first, count)
        hist.evict(s, first, count)
        evicted += count // P
    assert evicted > 0
    assert cache.page_list(0, 0)[1] == free0 + evicted
    for st in range(3):
        q = W.draw_q(w, 0, step=st).cuda()
        out = hist.append(cache, 0, [w.new_tokens] * w.num_seqs, step=(q, w.softmax_scale)).cpu().numpy()
    worst = check(cache, w, 0, hist, q, out, window=window, sinks=sinks, rope=rope, name=f"evict-{name}")
    _note(f"[paged evict] case={name} worst row rel err {worst:.3e}")
    cache.close()


def test_evict_rejects_bad_ranges():
    k = H.kvq()
    w, P, window, sinks, _ = CASES["llama_window"]
    cache = H.make_cache(w, extra=16, page_tokens=P, window=window, sinks=sinks)
    hist = Hist(w)
    prefill(cache, hist, 0, w.lengths)
    L = w.lengths[0]
    for first, count in ((P + 1, P), (P, P + 3), (0, P), (P, (L // P) * P), (L // P * P - P, P)):
        with pytest.raises(k.KVQError) as e:
            cache.evict(0, first, count)
        assert e.value.status == k.KVQ_ERR_ARG, (first, count)
    assert cache.lengths(0)[0] == L
    cc = H.make_cache(w, extra=16)
    with pytest.raises(k.KVQError) as e:
        cc.evict(0, P, P)
    assert e.value.status == k.KVQ_ERR_UNSUPPORTED
    cache.close()
    cc.close()


def test_reset_reuses_pages():
    w, P, _, _, _ = CASES["mixed"]
    cache = H.make_cache(w, extra=16, page_tokens=P)
    hist = Hist(w)
    prefill(cache, hist, 0, w.lengths)
    free0 = cache.page_list(0, 0)[1]
    held = sum(p != NO_PAGE for p in cache.page_list(0, 9)[0])
    cache.reset(9)
    hist.k[9], hist.v[9] = hist.k[9][:0], hist.v[9][:0]
    assert cache.page_list(0, 9)[1] == free0 + held and cache.lengths(0)[9] == 0
    counts = [0] * 9 + [333]
    hist.append(cache, 0, counts)
    q = W.draw_q(w, 0).cuda()
    out = cache.decode(0, q, w.softmax_scale).cpu().numpy()
    check(cache, w, 0, hist, q, out, name="reset")
    cache.close()


def test_pool_exhaustion_fails_before_writing():
    """An append that needs more pages than the pool has free fails with
    KVQ_ERR_CAPACITY and changes nothing; smaller appends still work."""
    k = H.kvq()
    w = CASES["llama"][0].scaled(lengths=(100, 100, 100))
    P = 64
    cache = H.make_cache(w, capacity=[1000] * 3, page_tokens=P, num_pages=7)
    hist = Hist(w)
    hist.append(cache, 0, [100, 100, 100])  # 2 pages each: 6 of 7
    before = cache.codes.clone()
    with pytest.raises(k.KVQError) as e:
        cache.append(0, torch.zeros((2 * 100, w.kv_heads, w.head_dim), dtype=w.torch_dtype, device="cuda"),
                     torch.zeros((2 * 100, w.kv_heads, w.head_dim), dtype=w.torch_dtype, device="cuda"),
                     [100, 100, 0])
    assert e.value.status == k.KVQ_ERR_CAPACITY
    torch.cuda.synchronize()
    assert cache.lengths(0) == [100, 100, 100] and torch.equal(before, cache.codes)
    assert cache.page_list(0, 0)[1] == 1
    hist.append(cache, 0, [20, 0, 0])  # fills page 1 of sequence 0 and takes no new page... then one
    hist.append(cache, 0, [40, 0, 0])
    q = W.draw_q(w, 0).cuda()
    out = cache.decode(0, q, w.softmax_scale).cpu().numpy()
    check(cache, w, 0, hist, q, out, name="exhaustion")
    cache.close()


def test_copy_sequence_paged_forks():
    """kvq_copy_sequence within one paged cache is a fork with shared pages;
    across two caches it is refused."""
    k = H.kvq()
    w, P, _, _, _ = CASES["llama"]
    w = w.scaled(lengths=(500, 10, 0))
    cache = H.make_cache(w, capacity=[600] * 3, page_tokens=P)
    hist = Hist(w)
    prefill(cache, hist, 0, w.lengths)
    cache.copy_sequence(2, cache, 0)
    hist.k[2], hist.v[2] = hist.k[0].copy(), hist.v[0].copy()
    assert cache.page_list(0, 2)[0][:7] == cache.page_list(0, 0)[0][:7]
    q = W.draw_q(w, 0).cuda()
    out = hist.append(cache, 0, [w.new_tokens] * 3, step=(q, w.softmax_scale)).cpu().numpy()
    check(cache, w, 0, hist, q, out, name="copy")
    other = H.make_cache(w, capacity=[600] * 3, page_tokens=P)
    with pytest.raises(k.KVQError) as e:
        other.copy_sequence(0, cache, 0)
    assert e.value.status == k.KVQ_ERR_UNSUPPORTED
    cache.close()
    other.close()
