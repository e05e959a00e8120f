"""The five benchmark workloads at full size, through the C ABI, in the calls
and launch configuration bench.py times: the whole cached prefix appended in
one call, then the decode step itself -- kvq_decode_step (the new tokens
appended and attended in one call; one launch where the single-query kernel
serves the cache) for the one-layer workloads, and kvq_quantize_append_layers
plus kvq_decode_attention_layers over all 12 layers for the GPT-2 shape --
with the library's default split sizes. Sampled (layer, seq, kv head) units
are checked against the CPU oracle computed for that unit alone: packed codes,
metadata and residual rows bit-exact, and the attention rows of the unit's
query heads within 2e-3 of the fp64 oracle over the quantized cache. Every
other unit is checked for what holds at any size: lengths advanced by the
append and finite outputs. Pools, workspace and outputs start poisoned."""

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


def _samples(w):
    """(layer, seq, kv head) units compared with the oracle."""
    last_l, last_s, last_h = w.layers - 1, w.num_seqs - 1, w.kv_heads - 1
    if w.name == "long-gqa":
        return [(0, 0, last_h)]  # one 262k-token head: about 10 s of oracle work
    if w.name == "mixed":
        seqs = []
        for pair in W.BIT_PAIRS_MIXED:  # the first sequence of every bit pair
            for s, b in enumerate(w.bits):
                if tuple(b) == tuple(pair):
                    seqs.append(s)
                    break
        seqs.append(int(np.argmax(w.lengths)))
        return [(0, s, h) for s in sorted(set(seqs)) for h in (0, last_h)]
    layers = sorted({0, last_l})
    seqs = sorted({0, last_s})
    heads = sorted({0, last_h})
    return [(l, s, h) for l in layers for s in seqs for h in heads]


@pytest.mark.parametrize("name,window,sinks,rope", [
    ("tiny", 0, 0, 0.0), ("gpt2-small", 0, 0, 0.0), ("llama2-7b", 0, 0, 0.0), ("long-gqa", 0, 0, 0.0),
    ("mixed", 0, 0, 0.0),
    # with a full-precision window of 128 recent tokens and 32 sinks (bench.py --window 128 --sinks 32)
    ("llama2-7b", 128, 32, 0.0), ("long-gqa", 128, 32, 0.0),
    # keys before the rotary embedding, rotated in the kernel (bench.py --rope-base 10000): positions to 262k
    ("long-gqa", 0, 0, 10000.0)])
def test_full_size_workload(name, window, sinks, rope):
    w = W.get(name)
    R = w.q_heads // w.kv_heads
    _note(f"[fullsize] {name}: S={w.num_seqs} L={w.layers} Hq={w.q_heads} Hkv={w.kv_heads} D={w.head_dim} "
          f"tokens={sum(w.lengths)} +{w.new_tokens}/seq window={window} sinks={sinks} rope={rope}")
    cache = H.make_cache(w, window=window, sinks=sinks, rope_base=rope)
    outs = {}
    counts = [w.new_tokens] * w.num_seqs
    if w.layers == 1:  # the bench step: kvq_decode_step
        prefix, new = H.history(w, 0, device="cuda")
        cache.append(0, prefix[0], prefix[1], prefix[2])
        q = W.draw_q(w, 0)
        out = cache.step(0, new[0], new[1], counts, q.cuda(), w.softmax_scale)
        torch.cuda.synchronize()
        outs[0] = (q, out.cpu().numpy())
        del prefix, new
    else:  # the bench step of a multi-layer model: one append and one decode call over all layers
        news = []
        for layer in range(w.layers):
            prefix, new = H.history(w, layer, device="cuda")
            cache.append(layer, prefix[0], prefix[1], prefix[2])
            news.append(new)
            del prefix
        kn = torch.stack([n[0] for n in news])
        vn = torch.stack([n[1] for n in news])
        cache.append_layers(0, kn, vn, counts)
        del news, kn, vn
        qs = [W.draw_q(w, layer) for layer in range(w.layers)]
        out = cache.decode_layers(0, w.layers, torch.stack(qs).cuda(), w.softmax_scale)
        torch.cuda.synchronize()
        out = out.cpu().numpy()
        for layer in range(w.layers):
            outs[layer] = (qs[layer], out[layer])
    for layer in range(w.layers):
        assert cache.lengths(layer) == [L + w.new_tokens for L in w.lengths]
        assert np.isfinite(outs[layer][1]).all(), (name, layer)
    _note(f"[fullsize] {name}: cache filled and decoded; checking {len(_samples(w))} sampled units")
    worst = 0.0
    by_layer = {}
    for layer, s, h in _samples(w):
        by_layer.setdefault(layer, []).append((s, h))
    for layer, units in by_layer.items():
        prefix, new = H.history(w, layer, device="cuda")  # the same seeded draw again
        q, out = outs[layer]
        for s, h in units:
            k, v = H.full_seq(prefix, new, s)
            enc = H.assert_head_bytes(cache, w, layer, s, h, k, v)
            if window or sinks:
                enc = H.encode_window(w, k, v, s, h, window, sinks)
            qs = q[s, h * R:(h + 1) * R].float().numpy().astype(np.float64)
            if rope:
                ref = o.attend_rope(qs, enc["k_hat"], enc["v_hat"], w.softmax_scale, rope)
            else:
                ref = o.attend_heads(qs, [enc["k_hat"]], [enc["v_hat"]], w.softmax_scale)
            err = H.row_rel_err(out[s, h * R:(h + 1) * R], ref)
            worst = max(worst, float(err.max()))
            assert np.all(err <= H.ATTN_TOL), (name, layer, s, h, float(err.max()))
        del prefix, new
    _note(f"[fullsize] {name}: worst row rel err {worst:.3e}")
    cache.close()
