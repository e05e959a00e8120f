"""Full-precision recent window and attention sinks on the GPU against the
CPU oracle: with a window of R tokens and S sink tokens the decode attention
reads the whole key blocks inside [S, len - R) quantized and every other
token in the input dtype ([U] "O Imposto dos Sistemas e Por Que Nao E um
Detalhe"; [U] "O Que Fazer Com Isso"; [U] "Onde o Trabalho Esta Indo").
Stored codes stay those of the plain cache; attention within 2e-3 of the
fp64 oracle over the windowed reconstruction; kvq_dequantize bit-exact."""

import sys

import numpy as np
import pytest
import torch

from bit_kv_cache_groupwise_amd import workloads as W
from oracle import kvq_oracle as o
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


# (workload, window, sinks): every decode kernel, block lengths 1, 32, 64 and 256,
# lengths below the sinks, inside the window and far past it
CASES = {
    # single-query kernel, head_dim 128, 2-bit, G = 32
    "llama": (W.llama2_7b().scaled(num_seqs=5, kv_heads=3, q_heads=3, lengths=(4096, 1000, 130, 20, 0),
                                   bits=((2, 2),) * 5), 128, 32),
    # single-query kernel, head_dim 64, K6/V4, G = 64, several layers
    "gpt2": (W.gpt2_small().scaled(num_seqs=3, layers=2, kv_heads=2, q_heads=2, lengths=(1024, 777, 64),
                                   bits=((6, 4),) * 3), 100, 64),
    # query-group kernel (16 per kv head), head_dim 256, bf16, K4/V8
    "gqa": (W.long_gqa().scaled(lengths=(3000,)), 128, 32),
    # query-group kernel over several bit pairs, lengths around the block edges
    "mixed": (W.mixed_batch().scaled(num_seqs=10, lengths=(0, 1, 31, 32, 33, 100, 512, 1000, 1500, 2047),
                                     bits=tuple(W.BIT_PAIRS_MIXED[i % 5] for i in range(10))), 64, 32),
    # generic split kernel: per-token keys (block of 1 token), sinks not a multiple of 32
    "ktoken": (W.gpt2_small().scaled(num_seqs=2, layers=1, kv_heads=2, q_heads=2, lengths=(300, 64),
                                     bits=((6, 4),) * 2, axis_k=o.AXIS_TOKEN), 50, 3),
    # generic split kernel: head_dim 32, fp32 input, 3-bit
    "d32": (W.tiny().scaled(head_dim=32, lengths=(395,), bits=((3, 3),)), 40, 32),
    # head_dims that do not divide 256 (generic split kernel), fp32 input, query groups of 2
    "d96": (W.tiny().scaled(head_dim=96, lengths=(300,), bits=((4, 4),)), 64, 32),
    "d160": (W.tiny().scaled(head_dim=160, kv_heads=2, q_heads=4, lengths=(200,), bits=((3, 4),)), 40, 0),
    # key blocks of 256 tokens, window only
    "bigG": (W.llama2_7b().scaled(num_seqs=2, kv_heads=2, q_heads=4, lengths=(1700, 256), group_k=256,
                                  group_v=128, bits=((4, 6), (8, 3))), 128, 0),
    # sinks only, no recent window beyond the residual
    "sinks_only": (W.llama2_7b().scaled(num_seqs=2, kv_heads=2, q_heads=2, lengths=(700, 40),
                                        bits=((2, 2),) * 2), 0, 64),
}


def _check(cache, w, layer, window, sinks, q, out, hist_k, hist_v, name):
    worst = 0.0
    for s in range(w.num_seqs):
        k, v = hist_k(s), hist_v(s)
        encs = []
        for h in range(w.kv_heads):
            H.assert_head_bytes(cache, w, layer, s, h, k, v)  # the stored codes do not depend on the window
            encs.append(H.encode_window(w, k, v, s, h, window, sinks))
        kd, vd = cache.dequantize(layer, s)
        torch.cuda.synchronize()
        for h in range(w.kv_heads):
            np.testing.assert_array_equal(kd[h].cpu().numpy(), encs[h]["k_hat"].astype(np.float32),
                                          err_msg=f"{name} k s{s} h{h}")
            np.testing.assert_array_equal(vd[h].cpu().numpy(), encs[h]["v_hat"].astype(np.float32),
                                          err_msg=f"{name} v s{s} h{h}")
        ref = H.attn_ref(w, q[s].float().cpu().numpy(), encs)
        err = H.row_rel_err(out[s], ref)
        worst = max(worst, float(err.max()))
        assert np.all(err <= H.ATTN_TOL), (name, s, err.max())
    return worst


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("chunks", [None, [1, 7, 100]], ids=["bulk", "chunked"])
def test_window_parity(name, chunks):
    """Prefill (in one append or in chunks that wrap the recent ring many
    times), then the decode step's tokens, then decode attention."""
    w, window, sinks = CASES[name]
    if chunks and name in ("gqa", "mixed", "llama"):
        w = w.scaled(lengths=tuple(min(L, 600) for L in w.lengths))
    layer = w.layers - 1
    _note(f"[window] case={name} chunks={chunks} R={window} S={sinks} lens={w.lengths}")
    cache = H.make_cache(w, window=window, sinks=sinks)
    prefix, new = H.history(w, layer)
    H.append_chunks(cache, layer, prefix[0], prefix[1], prefix[2], chunks)
    H.append_chunks(cache, layer, new[0], new[1], new[2])
    torch.cuda.synchronize()
    q = W.draw_q(w, layer)
    out = cache.decode(layer, q.cuda(), w.softmax_scale).cpu().numpy()
    worst = _check(cache, w, layer, window, sinks, q, out, lambda s: H.full_seq(prefix, new, s)[0],
                   lambda s: H.full_seq(prefix, new, s)[1], name)
    _note(f"[window] case={name} worst row rel err {worst:.3e}")
    cache.close()


def test_window_covering_the_cache_is_exact_attention():
    """A window longer than every sequence: the output is softmax attention over
    the unquantized rows (torch SDPA in float64 on the CPU)."""
    w = W.llama2_7b().scaled(num_seqs=2, kv_heads=2, q_heads=2, lengths=(300, 77), bits=((2, 2),) * 2)
    cache = H.make_cache(w, window=512)
    prefix, new = H.history(w, 0)
    H.append_chunks(cache, 0, prefix[0], prefix[1], prefix[2])
    H.append_chunks(cache, 0, new[0], new[1], new[2])
    q = W.draw_q(w, 0)
    out = cache.decode(0, q.cuda(), w.softmax_scale).cpu().numpy()
    for s in range(w.num_seqs):
        k, v = H.full_seq(prefix, new, s)
        for h in range(w.kv_heads):
            kk = torch.from_numpy(k[:, h].astype(np.float64))[None, None]
            vv = torch.from_numpy(v[:, h].astype(np.float64))[None, None]
            qq = q[s, h].double()[None, None, None]
            ref = torch.nn.functional.scaled_dot_product_attention(qq, kk, vv, scale=w.softmax_scale)[0, 0, 0]
            assert H.row_rel_err(out[s, h], ref.numpy()) <= H.ATTN_TOL
    cache.close()


@pytest.mark.parametrize("name", ["llama", "gqa", "ktoken"])
def test_window_decode_step_and_layers(name):
    """kvq_decode_step with a window (one fused launch for one query per kv head
    on the steps that complete no key block, where the workgroup that attends
    the window first copies the new rows into it) equals the two calls bit for
    bit; 40 steps cross key-block edges and the recent ring's wrap;
    kvq_decode_attention_layers over two layers equals the per-layer calls; the
    last step meets the oracle."""
    w, window, sinks = CASES[name]
    w = w.scaled(layers=2, lengths=tuple(min(L, 500) for L in w.lengths), new_tokens=1)
    _note(f"[window step] case={name} R={window} S={sinks}")
    steps = 40
    ca = H.make_cache(w, extra=steps, window=window, sinks=sinks)
    cb = H.make_cache(w, extra=steps, window=window, sinks=sinks)
    prefix = {l: H.history(w, l)[0] for l in range(2)}
    for c in (ca, cb):
        for l in range(2):
            c.append(l, prefix[l][0].cuda(), prefix[l][1].cuda(), prefix[l][2])
    ks, vs, cnts = [prefix[1][0]], [prefix[1][1]], [prefix[1][2]]
    counts = [1] * w.num_seqs
    for st in range(steps):
        kn, vn = W.draw_kv(w, 1, counts, device="cpu", stream=1 + st)
        q = W.draw_q(w, 1, step=st).cuda()
        for c in (ca, cb):  # layer 0 follows along
            c.append(0, kn.cuda(), vn.cuda(), counts)
        oa = ca.step(1, kn.cuda(), vn.cuda(), counts, q, w.softmax_scale)
        cb.append(1, kn.cuda(), vn.cuda(), counts)
        ob = cb.decode(1, q, w.softmax_scale)
        torch.cuda.synchronize()
        assert torch.equal(oa, ob), (name, st)
        ks.append(kn)
        vs.append(vn)
        cnts.append(counts)
    q2 = torch.stack([W.draw_q(w, 0, step=99), q.cpu()]).cuda()
    multi = ca.decode_layers(0, 2, q2, w.softmax_scale).cpu().numpy()
    for l in range(2):
        single = ca.decode(l, q2[l].contiguous(), w.softmax_scale).cpu().numpy()
        assert np.max(H.row_rel_err(multi[l], single)) < 2e-5, l
    out = oa.cpu().numpy()
    hk = lambda s: torch.cat([H.seq_rows(x, c, s) for x, c in zip(ks, cnts)]).float().numpy()
    hv = lambda s: torch.cat([H.seq_rows(x, c, s) for x, c in zip(vs, cnts)]).float().numpy()
    _check(ca, w, 1, window, sinks, q.cpu(), out, hk, hv, name)
    ca.close()
    cb.close()


def test_window_geometry_errors():
    """Sinks that are not whole key blocks, negative sizes and a window past the
    limit are rejected at plan time."""
    kvq = H.kvq()
    w = W.llama2_7b().scaled(num_seqs=1, kv_heads=1, q_heads=1, lengths=(10,), bits=((2, 2),))
    for window, sinks in ((0, 16), (-1, 0), (0, -32), (4096, 0), (3000, 1088)):
        with pytest.raises(kvq.KVQError) as e:
            kvq.kvq_plan(H.geom_of(w, window=window, sinks=sinks), [100], [2], [2])
        assert e.value.status == kvq.KVQ_ERR_ARG, (window, sinks)


def test_window_multi_layer_append():
    """kvq_quantize_append_layers with a window: every layer keeps its own window
    rows (prefix by per-layer appends, then 70 tokens into three layers in one
    call, more than the recent ring of 64 + 32 rows), and each layer's decode
    meets the oracle."""
    w = W.llama2_7b().scaled(num_seqs=2, kv_heads=2, q_heads=2, lengths=(300, 100), bits=((2, 2),) * 2,
                             new_tokens=70)
    L, window, sinks = 3, 64, 32
    cache = H.make_cache(w.scaled(layers=L), layers=L, window=window, sinks=sinks)
    hist = {l: H.history(w, l) for l in range(L)}
    for l in range(L):
        (kp, vp, cp), _ = hist[l]
        cache.append(l, kp.cuda(), vp.cuda(), cp)
    kn = torch.stack([hist[l][1][0] for l in range(L)]).cuda()
    vn = torch.stack([hist[l][1][1] for l in range(L)]).cuda()
    cache.append_layers(0, kn, vn, hist[0][1][2])
    for l in range(L):
        q = W.draw_q(w, l)
        out = cache.decode(l, q.cuda(), w.softmax_scale).cpu().numpy()
        prefix, new = hist[l]
        for s in range(w.num_seqs):
            k, v = H.full_seq(prefix, new, s)
            encs = [H.encode_window(w, k, v, s, h, window, sinks) for h in range(w.kv_heads)]
            ref = H.attn_ref(w, q[s].float().numpy(), encs)
            assert np.all(H.row_rel_err(out[s], ref) <= H.ATTN_TOL), (l, s)
    cache.close()


@pytest.mark.parametrize("window,sinks", [(0, 0), (64, 32)])
def test_copy_sequence(window, sinks):
    """kvq_copy_sequence forks a sequence (beam search, prefix reuse): the copy,
    within the cache and into a second cache, then takes further appends and
    decodes exactly as the source's history says; mismatches are rejected."""
    kvq = H.kvq()
    w = W.llama2_7b().scaled(num_seqs=3, kv_heads=2, q_heads=2, lengths=(300, 100, 300), bits=((2, 2),) * 3,
                             new_tokens=5)
    L = 2
    wl = w.scaled(layers=L)
    a = H.make_cache(wl, layers=L, extra=10, window=window, sinks=sinks)
    b = H.make_cache(wl, layers=L, extra=10, window=window, sinks=sinks)
    hist = {l: H.history(w, l) for l in range(L)}
    for l in range(L):
        (kp, vp, cp), _ = hist[l]
        a.append(l, kp.cuda(), vp.cuda(), cp)
    a.copy_sequence(2, a, 0)          # seq 2 of a becomes seq 0's history (it had its own)
    b.copy_sequence(2, a, 0, 1, 1)    # layer 1 of b's seq 2 as well
    assert a.lengths(0)[2] == 300 and a.lengths(1)[2] == 300 and b.lengths(1)[2] == 300 and b.lengths(0)[2] == 0
    for h in range(w.kv_heads):
        k, v = H.full_seq(hist[1][0], (hist[1][1][0][:0], hist[1][1][1][:0], [0] * 3), 0)
        H.assert_head_bytes(b, w, 1, 2, h, k, v)  # the copy into the second cache
    # then the same new tokens go to seq 0 and its fork
    for l in range(L):
        (kn, vn, _) = hist[l][1]
        kk = torch.cat([H.seq_rows(kn, [5] * 3, 0)] * 3).cuda()
        vv = torch.cat([H.seq_rows(vn, [5] * 3, 0)] * 3).cuda()
        a.append(l, kk, vv, [5, 0, 5])
    for l in range(L):
        prefix, new = hist[l]
        k, v = H.full_seq(prefix, new, 0)
        q = W.draw_q(w, l)
        q[2] = q[0]
        out = a.decode(l, q.cuda(), w.softmax_scale).cpu().numpy()
        np.testing.assert_array_equal(out[2], out[0])
        for h in range(w.kv_heads):
            H.assert_head_bytes(a, w, l, 2, h, k, v)  # the fork's stored bytes: seq 0's history
        if window or sinks:
            encs = [H.encode_window(w, k, v, 0, h, window, sinks) for h in range(w.kv_heads)]
        else:
            encs = [H.encode(w, k, v, 0, h) for h in range(w.kv_heads)]
        ref = H.attn_ref(w, q[0].float().numpy(), encs)
        assert np.all(H.row_rel_err(out[2], ref) <= H.ATTN_TOL), l
    for args, st in (((2, a, 2), kvq.KVQ_ERR_ARG), ((3, a, 0), kvq.KVQ_ERR_ARG), ((0, a, 0, 1, 2), kvq.KVQ_ERR_ARG)):
        with pytest.raises(kvq.KVQError) as e:
            a.copy_sequence(*args)
        assert e.value.status == st
    other = H.make_cache(wl, layers=L, extra=11, window=window, sinks=sinks)  # capacities differ
    with pytest.raises(kvq.KVQError) as e:
        other.copy_sequence(0, a, 0)
    assert e.value.status == kvq.KVQ_ERR_ARG
    for c in (a, b, other):
        c.close()
