#!/usr/bin/env python3
"""Error budget of groupwise KV-cache quantization on synthetic caches.

How far the stored tensors, the attention logits and the attention output of a
decode step move from their unquantized values, for the four key/value axis
combinations and for a sweep of group sizes and bit widths. The quantized
cache is built and read by the library on the GPU (kvq_quantize_append,
kvq_dequantize, and the fused kvq_decode_attention where it applies); the
unquantized reference is plain float64 softmax attention over the input rows.

Why the output and not only the tensors: a value cache is never read by
itself but through the attention-weighted sum over tokens, so its error has to
be measured at the attention output, where a per-channel value grouping can be
far worse than a per-token one even when its reconstruction error is smaller
([U] "Valores: Onde a Intuicao Quebra"; keys and their fixed outlier channels:
[U] "Chaves: Os Valores Extremos Vivem em Canais Fixos"; the per-element bound
of half a step: [U] "O Que o Erro de Quantizacao E Realmente Feito"). Group
granularity (whole vector, per head, 64, 32 channels) is the other lever
([H] "Asymetrie kvantizace KV cache", the granularity comparison), and so is a
full-precision window of recent tokens plus attention-sink tokens ([U] "O
Imposto dos Sistemas e Por Que Nao E um Detalhe", "O Que Fazer Com Isso"),
which the library reads unquantized.

Inputs: the Llama-2-7B-shaped recipe of bench.py (key channel magnitudes
lognormal(0, 1), 1% of channels 20x; queries N(0,1)), 4 sequences of 2048
tokens, 8 heads of 128 channels, fp16; values either flat N(0,1) or with a
lognormal per-token scale. Prints one JSON line per configuration and a
markdown table.
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

CH, TOK = 0, 1
AXIS_NAME = {CH: "channel", TOK: "token"}


def rel_err(a, b):
    """||a - b|| / ||b|| over all elements (float64)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    nb = np.linalg.norm(b)
    return float(np.linalg.norm(a - b) / nb) if nb > 0 else float(np.linalg.norm(a))


def softmax_attention(q, k, v, scale):
    """float64 attention of one query per head. q [H][D], k and v [H][T][D]
    -> (out [H][D], logits [H][T], weights [H][T])."""
    q = np.asarray(q, np.float64)
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    logits = np.einsum("hd,htd->ht", q, k) * scale
    w = np.exp(logits - logits.max(axis=1, keepdims=True))
    w /= w.sum(axis=1, keepdims=True)
    return np.einsum("ht,htd->hd", w, v), logits, w


def top_mass(weights, frac=0.05):
    """Share of the attention mass held by the top `frac` of tokens (mean over rows)."""
    w = np.sort(np.asarray(weights, np.float64), axis=1)[:, ::-1]
    n = max(1, int(math.ceil(frac * w.shape[1])))
    return float(np.mean(w[:, :n].sum(axis=1)))


def recent_queries(k, S, T, H, D, gen):
    """Queries that attend to the most recent tokens: per (sequence, head), the
    sum of the last 8 keys scaled to norm 4*sqrt(D), plus N(0,1) noise. A stand-in
    for decode steps whose attention concentrates on recent tokens, the case the
    full-precision window targets ([U] "O Imposto dos Sistemas ..."); synthetic,
    not a trained model's queries."""
    import torch
    kk = k.float().reshape(S, T, H, D)[:, T - 8:].sum(dim=1)  # [S][H][D]
    kk = kk / kk.norm(dim=-1, keepdim=True) * (4.0 * D ** 0.5)
    return kk + torch.randn(kk.shape, generator=gen, device=k.device)


def run_config(w, device="cuda", window=0, sinks=0, q_recent=False, whole_vector=False):
    """Quantize w's cache on the GPU, read it back and decode; return the error
    metrics. With a window or sinks, the reconstruction read back is the one the
    attention reads (those tokens unquantized). q_recent: queries from
    recent_queries instead of N(0,1). whole_vector: groups that span every kv
    head of a token (token axis, group = kv_heads * head_dim): the cache is
    built as one head of kv_heads * head_dim channels (the same [T][H][D] rows),
    and its reconstruction is split back into heads for the attention; no fused
    decode (it would attend over the merged head)."""
    import torch

    from bit_kv_cache_groupwise_amd import kvq
    from bit_kv_cache_groupwise_amd import workloads as W

    S, H, D, T = w.num_seqs, w.kv_heads, w.head_dim, w.lengths[0]
    Hc, Dc = (1, H * D) if whole_vector else (H, D)
    geom = kvq.geometry(layers=1, num_seqs=S, kv_heads=Hc, q_heads=Hc if whole_vector else w.q_heads, head_dim=Dc,
                        group_k=Dc if whole_vector else w.group_k, group_v=Dc if whole_vector else w.group_v,
                        axis_k=TOK if whole_vector else w.axis_k, axis_v=TOK if whole_vector else w.axis_v,
                        in_dtype=w.in_dtype, window=window, sinks=sinks)
    cache = kvq.Cache(geom, list(w.lengths), [b[0] for b in w.bits], [b[1] for b in w.bits], device=device)
    k, v = W.draw_kv(w, 0, w.lengths, device=device, stream=0)
    cache.append(0, k.reshape(-1, Hc, Dc), v.reshape(-1, Hc, Dc), list(w.lengths))
    q = W.draw_q(w, 0, device=device)
    if q_recent:
        gen = torch.Generator(device=device)
        gen.manual_seed(4242)
        q = recent_queries(k, S, T, H, D, gen).to(q.dtype)
    fused = None
    if not whole_vector:
        fused = cache.decode(0, q, w.softmax_scale).double().cpu().numpy()
    torch.cuda.synchronize()
    kx = k.double().cpu().numpy().reshape(S, T, H, D).transpose(0, 2, 1, 3)  # [S][H][T][D]
    vx = v.double().cpu().numpy().reshape(S, T, H, D).transpose(0, 2, 1, 3)
    qx = q.double().cpu().numpy()
    acc = {"k_recon": [], "v_recon": [], "logit_rms": [], "logit_max": [], "out_deq": [], "out_fused": [],
           "out_deq_max": [], "top5_mass": []}
    kn2 = kd2 = vn2 = vd2 = 0.0
    for s in range(S):
        kd, vd = cache.dequantize(0, s)
        # [Hc][T][Dc] -> [H][T][D] (a no-op unless whole_vector)
        kd = kd.double().cpu().numpy().reshape(Hc, T, Dc).transpose(1, 0, 2).reshape(T, H, D).transpose(1, 0, 2)
        vd = vd.double().cpu().numpy().reshape(Hc, T, Dc).transpose(1, 0, 2).reshape(T, H, D).transpose(1, 0, 2)
        kn2 += float(np.sum(kx[s] ** 2))
        kd2 += float(np.sum((kd - kx[s]) ** 2))
        vn2 += float(np.sum(vx[s] ** 2))
        vd2 += float(np.sum((vd - vx[s]) ** 2))
        o_ref, lg_ref, w_ref = softmax_attention(qx[s], kx[s], vx[s], w.softmax_scale)
        o_deq, lg_deq, _ = softmax_attention(qx[s], kd, vd, w.softmax_scale)
        dl = lg_deq - lg_ref
        acc["logit_rms"].append(float(np.sqrt(np.mean(dl ** 2)) / np.std(lg_ref)))
        acc["logit_max"].append(float(np.max(np.abs(dl))))
        per_row = np.linalg.norm(o_deq - o_ref, axis=1) / np.linalg.norm(o_ref, axis=1)
        acc["out_deq"].append(float(np.mean(per_row)))
        acc["out_deq_max"].append(float(np.max(per_row)))
        if fused is not None:
            acc["out_fused"].append(float(np.mean(np.linalg.norm(fused[s] - o_ref, axis=1)
                                                  / np.linalg.norm(o_ref, axis=1))))
        acc["top5_mass"].append(top_mass(w_ref))
    cache.close()
    return {
        "axis_k": AXIS_NAME[TOK if whole_vector else w.axis_k], "axis_v": AXIS_NAME[TOK if whole_vector else w.axis_v],
        "group_k": "vector" if whole_vector else w.group_k, "group_v": "vector" if whole_vector else w.group_v,
        "bits": list(w.bits[0]), "v_dist": w.v_dist, "window": window, "sinks": sinks,
        "queries": "recent" if q_recent else "normal",
        "k_recon_rel": math.sqrt(kd2 / kn2), "v_recon_rel": math.sqrt(vd2 / vn2),
        "logit_rms_over_std": float(np.mean(acc["logit_rms"])), "logit_max_abs": float(np.max(acc["logit_max"])),
        "out_rel_dequant": float(np.mean(acc["out_deq"])), "out_rel_dequant_max": float(np.max(acc["out_deq_max"])),
        "out_rel_fused": float(np.mean(acc["out_fused"])) if acc["out_fused"] else None,
        "top5pct_attention_mass": float(np.mean(acc["top5_mass"])),
    }


def configs(T=2048):
    from bit_kv_cache_groupwise_amd import workloads as W

    base = W.llama2_7b().scaled(name="error-budget", num_seqs=4, kv_heads=8, q_heads=8, lengths=(T,) * 4)
    out = []
    # the four axis combinations at 32-element groups
    for bits in (2, 4):
        for v_dist in ("normal", "token_lognormal"):
            for ak in (CH, TOK):
                for av in (TOK, CH):
                    out.append(base.scaled(axis_k=ak, axis_v=av, group_k=32, group_v=32, bits=((bits, bits),) * 4,
                                           v_dist=v_dist))
    # group-size sweep for keys per channel and values per token (128 = one head's channels)
    for bits in (2, 4):
        for G in (64, 128):
            out.append(base.scaled(group_k=G, group_v=G, bits=((bits, bits),) * 4, v_dist="token_lognormal"))
        out.append(base.scaled(group_k=256, group_v=128, bits=((bits, bits),) * 4, v_dist="token_lognormal"))
    return [(x, 0, 0, False, False) for x in out] + window_configs(base) + granularity_configs(T)


def granularity_configs(T=2048):
    """Scales per whole vector, per head, per 64 and per 32 channels ([H]
    "Granularita jako jediné univerzální doporučení"; [H] "Výchozí zjištění na
    GPT-2": per-head against whole-vector scaling): keys and values both grouped
    along the channels of a token, 3 and 4 bits, two kv heads of 128 channels
    (a 256-channel vector)."""
    from bit_kv_cache_groupwise_amd import workloads as W

    base = W.llama2_7b().scaled(name="granularity", num_seqs=4, kv_heads=2, q_heads=2, lengths=(T,) * 4,
                                axis_k=TOK, axis_v=TOK, v_dist="token_lognormal")
    rows = []
    for bits in (3, 4):
        wb = base.scaled(bits=((bits, bits),) * 4)
        rows.append((wb.scaled(group_k=128, group_v=128), 0, 0, False, True))  # whole vector
        for G in (128, 64, 32):  # per head, then finer
            rows.append((wb.scaled(group_k=G, group_v=G), 0, 0, False, False))
    return rows


def window_configs(base):
    """Full-precision recent window and sinks at 2 bits (keys per channel,
    values per token, groups of 32): (workload, window, sinks)."""
    w2 = base.scaled(group_k=32, group_v=32, bits=((2, 2),) * 4, v_dist="token_lognormal")
    rows = [(w2, win, snk, False, False) for win, snk in ((32, 0), (128, 0), (512, 0), (128, 32), (0, 64))]
    # queries that attend to the most recent tokens
    return rows + [(w2, win, snk, True, False) for win, snk in ((0, 0), (32, 0), (128, 0), (128, 32))]


def table(rows):
    lines = ["| K axis | V axis | G (K, V) | bits | window, sinks | V recipe | queries | K recon | V recon "
             "| logit rms/std | out (dequant) | out (fused) | top-5% mass |",
             "|---|---|---|---|---|---|---|---|---|---|---|---|---|"]
    for r in rows:
        fused = f"{r['out_rel_fused']:.2e}" if r["out_rel_fused"] is not None else "—"
        lines.append(f"| {r['axis_k']} | {r['axis_v']} | {r['group_k']}, {r['group_v']} | {r['bits'][0]} | "
                     f"{r['window']}, {r['sinks']} | "
                     f"{r['v_dist']} | {r['queries']} | "
                     f"{r['k_recon_rel']:.3e} | {r['v_recon_rel']:.3e} | "
                     f"{r['logit_rms_over_std']:.3e} | {r['out_rel_dequant']:.3e} | {fused} | "
                     f"{r['top5pct_attention_mass']:.2f} |")
    return "\n".join(lines)


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--tokens", type=int, default=2048)
    args = ap.parse_args()
    rows = []
    for w, window, sinks, q_recent, whole in configs(args.tokens):
        r = run_config(w, window=window, sinks=sinks, q_recent=q_recent, whole_vector=whole)
        rows.append(r)
        print(json.dumps(r), flush=True)
    print(table(rows), flush=True)


if __name__ == "__main__":
    main()
