#!/usr/bin/env python3
"""Decode-step benchmark of the quantized KV cache on one MI355X.

One step = the new tokens of every sequence appended into one layer, then
decode attention over that layer (every cached token, the new ones included),
as one kvq_decode_step call (--unfused-step: kvq_quantize_append then
kvq_decode_attention). The default workload is the largest single-GPU
configuration, the mixed batch: 64 sequences with lengths uniform in
[512, 32768], 64 query heads over 8 kv heads of 128 channels, fp16,
per-sequence (K, V) bits from {(2,2),(3,3),(4,4),(6,4),(4,8)}, groups of 32,
16 new tokens per sequence per step (so about half the sequences complete a
key block on every step). Independent layer caches are rotated where one
layer is smaller than 4x the 256 MB last-level cache, and the timed steps
cover whole key-block cycles of every rotated cache. A multi-layer workload
(the GPT-2 shape, 12 layers) appends into all of them in one
kvq_quantize_append_layers call and decodes them in one
kvq_decode_attention_layers call (--per-layer-decode: one of each per layer).

Prints one JSON line: metric/value (decode-step GB/s of algorithmic bytes),
tokens/s, the step's roofline (HIP events on the launch stream, a separate
loop of at least 20 event-bracketed steps after the wall-clock region) and
the CPU oracle timed on the host (one core, and all allowed cores).
"""

from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBPS = 8000.0  # MI355X HBM3E, published
LLC_BYTES = 256 << 20  # MI355X Infinity Cache

METRIC = "quantized decode-attention HBM GB/s (% of peak) and tokens/s; quantize GB/s"


def algorithmic_head_bytes(T, D, axis_k, axis_v, Gk, Gv, bk, bv, ib, window=0, sinks=0):
    """Bytes decode attention must read for one (seq, kv head) at length T:
    packed codes + 4-byte (step, zero) pairs + residual rows in the input dtype.
    With a full-precision window or sinks: the codes and pairs of the whole key
    blocks inside [sinks, T - window), and every other token's key and value
    rows in the input dtype."""
    if window or sinks:
        blk = max([G for axis, G in ((axis_k, Gk), (axis_v, Gv)) if axis == 0] or [1])
        q = max(sinks, blk * ((T - window) // blk))
        nq = max(0, q - sinks)
        tot = 2 * (T - nq) * D * ib
        for axis, G, B in ((axis_k, Gk, bk), (axis_v, Gv, bv)):
            tot += nq * D * B // 8 + (nq // G * D if axis == 0 else nq * (D // G)) * 4
        return tot
    tot = 0
    for axis, G, B in ((axis_k, Gk, bk), (axis_v, Gv, bv)):
        if axis == 0:
            tq = T // G * G
            tot += tq * D * B // 8 + (tq // G) * D * 4 + (T - tq) * D * ib
        else:
            tot += T * D * B // 8 + T * (D // G) * 4
    return tot


def rotation_for(step_bytes):
    """Independent layer caches to cycle through so that a step never reads a
    warm cache: 4x the last-level cache, capped where a step is too small for
    HBM to matter (the small configurations are latency-bound)."""
    return max(1, min(64, math.ceil(4 * LLC_BYTES / max(step_bytes, 1))))


def main():
    ap = argparse.ArgumentParser(description=__doc__.splitlines()[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=0,
                    help="timed steps (0: 50, or more so that every rotated cache completes a key-block cycle)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="mixed",
                    choices=["tiny", "gpt2-small", "llama2-7b", "long-gqa", "mixed"])
    ap.add_argument("--rotate", type=int, default=0, help="independent layer caches to cycle through (0 = auto)")
    ap.add_argument("--per-layer-decode", action="store_true",
                    help="multi-layer workloads: one append and one decode call per layer instead of one each for all layers")
    ap.add_argument("--unfused-step", action="store_true",
                    help="single-layer workloads: kvq_quantize_append then kvq_decode_attention instead of "
                         "kvq_decode_step")
    ap.add_argument("--event-steps", type=int, default=0,
                    help="steps of the event-timed loop after the wall-clock region (0: max(20, steps)); each "
                         "step's decode call is bracketed by a HIP event pair on the launch stream")
    ap.add_argument("--no-append-timing", action="store_true",
                    help="skip the separately timed appends after the timed region (profiled runs: every append "
                         "after the prefill then belongs to a timed decode step)")
    ap.add_argument("--window", type=int, default=0,
                    help="recent tokens kept in full precision (the decode reads them unquantized)")
    ap.add_argument("--sinks", type=int, default=0, help="first tokens kept in full precision")
    ap.add_argument("--rope-base", type=float, default=0.0,
                    help="keys cached before the rotary embedding with this base, rotated inside the decode (0: off)")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-sample-seconds", type=float, default=10.0,
                    help="CPU seconds per oracle leg (one core; all cores)")
    ap.add_argument("--cpu-workers", type=int, default=0,
                    help="processes of the all-core oracle leg (0: min(cpu count, 16))")
    ap.add_argument("--probe-reps", type=int, default=30, help="timed repetitions of the streaming-read probe")
    ap.add_argument("--copy-probe-mib", type=int, default=256,
                    help="plain device copy of this size before timing (calibrates HBM byte counters); 0 = none")
    args = ap.parse_args()
    if args.gpus != 1:
        print("bench.py runs on one GPU: this build has no multi-GPU path (use --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch

    from bit_kv_cache_groupwise_amd import workloads as W

    w = W.get(args.workload)
    # The CPU oracle first: its worker processes are forked before this process
    # touches the GPU.
    cpu = None if args.no_cpu_baseline else cpu_baseline(w, args.cpu_sample_seconds, args.window, args.sinks,
                                                         args.cpu_workers)

    from bit_kv_cache_groupwise_amd import kvq

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    ib = 4 if w.in_dtype == "f32" else 2
    S, H, D = w.num_seqs, w.kv_heads, w.head_dim
    n_new = w.new_tokens
    model_layers = w.layers  # layers attended per step (12 for the GPT-2 shape, else 1)
    step_lens = [L + n_new for L in w.lengths]
    WS = dict(window=args.window, sinks=args.sinks)
    step_bytes = sum(algorithmic_head_bytes(T, D, w.axis_k, w.axis_v, w.group_k, w.group_v, bk, bv, ib, **WS) * H
                     for T, (bk, bv) in zip(step_lens, w.bits)) * model_layers
    rot = args.rotate or rotation_for(step_bytes)
    # a key block of the cache in tokens; a rotated cache completes one every `cycle` of its appends
    blk = max([G for axis, G in ((w.axis_k, w.group_k), (w.axis_v, w.group_v)) if axis == 0] or [1])
    cycle = max(1, math.ceil(blk / n_new))
    steps = args.steps or max(50, rot * cycle)
    event_steps = args.event_steps or max(20, steps)
    append_timing_steps = 0 if args.no_append_timing else min(10, steps)
    total_steps = args.warmup + steps + event_steps + append_timing_steps
    appends_per_layer = math.ceil(total_steps / rot) + 1
    layers = rot * model_layers
    cap = [L + n_new * appends_per_layer for L in w.lengths]
    geom = kvq.geometry(layers=layers, num_seqs=S, kv_heads=H, q_heads=w.q_heads, head_dim=D, group_k=w.group_k,
                        group_v=w.group_v, axis_k=w.axis_k, axis_v=w.axis_v, in_dtype=w.in_dtype,
                        window=args.window, sinks=args.sinks, rope_base=args.rope_base)
    cache = kvq.Cache(geom, cap, [b[0] for b in w.bits], [b[1] for b in w.bits], device=dev)
    decode_kernel = {kvq.KVQ_DECODE_SINGLE_QUERY: "single_query", kvq.KVQ_DECODE_QUERY_GROUP: "query_group",
                     kvq.KVQ_DECODE_GENERIC: "generic"}[cache.decode_kernel()]

    # ---- bulk prefill = quantize-append into an empty cache (timed: quantize GB/s).
    # The append kernel runs once on a small scratch cache first (its first launch
    # in a process also loads the code); the first layer's prefill is timed three
    # times, emptied in between (kvq_reset_sequence), the median reported. A
    # multi-layer model (the 12-layer GPT-2 shape) prefills all of its layers in
    # one kvq_quantize_append_layers call, the shape of its decode step.
    qz_ms = []
    ev = lambda: torch.cuda.Event(enable_timing=True)
    warm = kvq.Cache(kvq.geometry(layers=1, num_seqs=S, kv_heads=H, q_heads=w.q_heads, head_dim=D,
                                  group_k=w.group_k, group_v=w.group_v, axis_k=w.axis_k, axis_v=w.axis_v,
                                  in_dtype=w.in_dtype), [w.group_k + 1] * S, [b[0] for b in w.bits],
                     [b[1] for b in w.bits], device=dev)
    wk, wv = W.draw_kv(w, 0, [w.group_k + 1] * S, device=dev, stream=0)
    warm.append(0, wk, wv, [w.group_k + 1] * S)
    torch.cuda.synchronize()
    warm.close()
    del warm, wk, wv
    for l0 in range(0, layers, model_layers):
        kv = [W.draw_kv(w, l % model_layers if rot == 1 else l, w.lengths, device=dev, stream=0)
              for l in range(l0, l0 + model_layers)]
        if model_layers > 1:
            k, v = torch.stack([x[0] for x in kv]), torch.stack([x[1] for x in kv])
        else:
            k, v = kv[0]
        del kv
        for rep in range(3 if l0 == 0 else 1):
            if rep:
                for s_ in range(S):
                    cache.reset(s_, l0, model_layers)
            torch.cuda.synchronize()
            e0, e1 = ev(), ev()
            e0.record()
            if model_layers > 1:
                cache.append_layers(l0, k, v, list(w.lengths))
            else:
                cache.append(l0, k, v, list(w.lengths))
            e1.record()
            torch.cuda.synchronize()
            qz_ms.append(e0.elapsed_time(e1))
        del k, v
    prefill_tokens = sum(w.lengths) * model_layers
    qz_bytes = model_layers * sum(H * append_head_bytes(0, T, D, w, bk, bv, ib)
                                  for T, (bk, bv) in zip(w.lengths, w.bits))
    quantize_gbps = qz_bytes / (np.median(qz_ms) * 1e-3) / 1e9

    # ---- calibration copy: a plain device-to-device copy of known size whose
    # FETCH_SIZE / WRITE_SIZE counters scale the decode kernel's (see profiles/)
    if args.copy_probe_mib:
        src = torch.empty(args.copy_probe_mib << 18, dtype=torch.float32, device=dev).fill_(1.0)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    # ---- per-step inputs, drawn up front. A multi-layer step decodes all its
    # layers in one kvq_decode_attention_layers call (one query per layer).
    multi = model_layers > 1 and not args.per_layer_decode
    fused_step = model_layers == 1 and not args.unfused_step
    dec_per_step = 1 if multi else model_layers
    new_k, new_v, qs = [], [], []
    for st in range(total_steps):
        if multi:
            kv = [W.draw_kv(w, m, [n_new] * S, device=dev, stream=1 + st) for m in range(model_layers)]
            new_k.append(torch.stack([x[0] for x in kv]))
            new_v.append(torch.stack([x[1] for x in kv]))
            del kv
        else:
            k, v = W.draw_kv(w, 0, [n_new] * S, device=dev, stream=1 + st)
            new_k.append(k)
            new_v.append(v)
        if multi:
            qs.append(torch.stack([W.draw_q(w, m, device=dev, step=st) for m in range(model_layers)]))
        else:
            qs.append(W.draw_q(w, 0, device=dev, step=st))
    out = torch.empty(((model_layers,) if multi else ()) + (S, w.q_heads, D), dtype=torch.float32, device=dev)
    ws = cache.workspace(model_layers if multi else 1)
    counts = [n_new] * S
    scale = w.softmax_scale

    # arguments marshalled once, as a serving loop would
    stream = torch.cuda.current_stream(dev).cuda_stream
    counts_c = kvq._i32(counts)
    kp = [t.data_ptr() for t in new_k]
    vp = [t.data_ptr() for t in new_v]
    qp = [t.data_ptr() for t in qs]
    out_p, ws_p, ws_b = out.data_ptr(), ws.data_ptr(), ws.numel()

    def step(st, dec_events=None, app_events=None):
        base = (st % rot) * model_layers
        if multi:
            if app_events is not None:
                app_events[0][0].record()
            kvq.kvq_quantize_append_layers(cache.handle, base, model_layers, kp[st], vp[st], counts_c, stream)
            if app_events is not None:
                app_events[0][1].record()
            if dec_events is not None:
                dec_events[0][0].record()
            kvq.kvq_decode_attention_layers(cache.handle, base, model_layers, qp[st], scale, out_p, ws_p, ws_b, stream)
            if dec_events is not None:
                dec_events[0][1].record()
            return
        if fused_step and app_events is None:
            # kvq_decode_step: the append and the attention in one call
            if dec_events is not None:
                dec_events[0][0].record()
            kvq.kvq_decode_step(cache.handle, base, kp[st], vp[st], counts_c, qp[st], scale, out_p, ws_p, ws_b,
                                stream)
            if dec_events is not None:
                dec_events[0][1].record()
            return
        for m in range(model_layers):
            l = base + m
            if app_events is not None:
                app_events[m][0].record()
            kvq.kvq_quantize_append(cache.handle, l, kp[st], vp[st], counts_c, stream)
            if app_events is not None:
                app_events[m][1].record()
            if dec_events is not None:
                dec_events[m][0].record()
            kvq.kvq_decode_attention(cache.handle, l, qp[st], scale, out_p, ws_p, ws_b, stream)
            if dec_events is not None:
                dec_events[m][1].record()

    # host mirror of the lengths, for the algorithmic bytes of every call
    lens = {l: list(w.lengths) for l in range(layers)}

    def account(st):
        """(decode bytes, append bytes) of step st's calls, per decode call; advances the mirror."""
        base = (st % rot) * model_layers
        dec, app = [], []
        for m in range(model_layers):
            l = base + m
            app.append(sum(H * append_head_bytes(L, n_new, D, w, bk, bv, ib) for L, (bk, bv) in
                           zip(lens[l], w.bits)))
            lens[l] = [x + n_new for x in lens[l]]
            dec.append(sum(algorithmic_head_bytes(T, D, w.axis_k, w.axis_v, w.group_k, w.group_v, bk, bv, ib,
                                                  **WS) * H for T, (bk, bv) in zip(lens[l], w.bits)))
        if args.window or args.sinks:  # the new rows are also copied into the full-precision window
            app = [a + S * n_new * H * 4 * D * ib for a in app]
        if multi:
            return [sum(dec)], [sum(app)]
        return dec, app

    for st in range(args.warmup):
        step(st)
        account(st)
    torch.cuda.synchronize()
    # ---- the timed region: `steps` steps, wall clock, no events
    t0 = time.perf_counter()
    for i in range(steps):
        step(args.warmup + i)
    torch.cuda.synchronize()
    wall_s = time.perf_counter() - t0
    dec_bytes, app_bytes = [], []
    for i in range(steps):
        d, a = account(args.warmup + i)
        dec_bytes.extend(d)
        app_bytes.extend(a)
    # ---- the event-timed loop: every step's decode call bracketed on the launch stream
    base_st = args.warmup + steps
    evs = [[[ev(), ev()] for _ in range(dec_per_step)] for _ in range(event_steps)]
    for j in range(event_steps):
        step(base_st + j, dec_events=evs[j])
    torch.cuda.synchronize()
    dec_ms = [evs[j][m][0].elapsed_time(evs[j][m][1]) for j in range(event_steps) for m in range(dec_per_step)]
    ev_bytes = []
    for j in range(event_steps):
        d, a = account(base_st + j)
        ev_bytes.extend([x + y for x, y in zip(d, a)] if fused_step else d)
    # ---- the append alone, for its latency
    base_st += event_steps
    aevs = [[[ev(), ev()] for _ in range(dec_per_step)] for _ in range(append_timing_steps)]
    for j in range(append_timing_steps):
        step(base_st + j, app_events=aevs[j])
        account(base_st + j)
    torch.cuda.synchronize()
    app_ms = [aevs[j][m][0].elapsed_time(aevs[j][m][1]) for j in range(append_timing_steps) for m in range(dec_per_step)]

    ms_per_step = wall_s * 1e3 / steps
    step_total_bytes = (sum(dec_bytes) + sum(app_bytes)) / steps
    value = step_total_bytes / (ms_per_step * 1e-3) / 1e9
    call_bytes = [x + y for x, y in zip(dec_bytes, app_bytes)] if fused_step else dec_bytes
    dec_avg_ms = float(np.mean(dec_ms))
    p10, p50, p90 = (float(x) * 1e3 for x in np.percentile(dec_ms, [10, 50, 90]))

    # ---- measured read ceiling: the library's plain streaming-read probe over
    # the byte count of one decode call, timed the same way (one event pair on
    # the launch stream) and kept cold by cycling through windows of a buffer
    # at least 4x the last-level cache
    probe_bytes = int(np.mean(call_bytes)) // 16 * 16
    win = (probe_bytes + 4095) // 4096 * 4096
    nwin = max(8, math.ceil(4 * LLC_BYTES / win))
    pbuf = torch.empty(win * nwin, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    probe_ms = []
    for r in range(args.probe_reps + 2):
        e0, e1 = ev(), ev()
        e0.record()
        kvq.kvq_read_probe(pbuf.data_ptr() + (r % nwin) * win, probe_bytes, sink.data_ptr(), stream)
        e1.record()
        torch.cuda.synchronize()
        if r >= 2:
            probe_ms.append(e0.elapsed_time(e1))
    del pbuf
    ceiling_gbps = probe_bytes / (float(np.median(probe_ms)) * 1e-3) / 1e9
    dec_gbps = float(np.mean(ev_bytes)) / (dec_avg_ms * 1e-3) / 1e9
    tokens_per_s = S * n_new / (ms_per_step * 1e-3)

    result = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.in_dtype,
        "accumulate": "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "num_seqs": S, "kv_heads": H, "q_heads": w.q_heads, "head_dim": D,
                   "cached_tokens": (list(sorted(set(w.lengths)))[:4] + ["..."] if len(set(w.lengths)) > 4 else
                                     sorted(set(w.lengths))) if len(set(w.lengths)) > 1 else w.lengths[0],
                   "cached_tokens_total": sum(w.lengths), "new_tokens_per_seq": n_new,
                   "layers_per_step": model_layers, "decode_calls_per_step": dec_per_step,
                   "bits_kv": sorted(set(w.bits)), "group": [w.group_k, w.group_v],
                   "input_dtype": w.in_dtype, "rotated_layer_caches": rot, "parallelism": "single-gpu",
                   "decode_kernel": decode_kernel,
                   **({"full_precision_window": args.window, "sinks": args.sinks} if args.window or args.sinks
                      else {}), **({"rope_base": args.rope_base} if args.rope_base else {})},
        "pct_of_hbm_peak": round(100 * value / HBM_PEAK_GBPS, 2),
        "tokens_per_s": round(tokens_per_s, 1),
        "decode_step_bytes": int(step_total_bytes),
        "decode_attention_GBps": round(dec_gbps, 2),
        "decode_call_us": round(dec_avg_ms * 1e3, 3),
        "decode_call_us_p10_p50_p90": [round(p10, 3), round(p50, 3), round(p90, 3)],
        "event_samples": len(dec_ms),
        "append_us": round(float(np.mean(app_ms)) * 1e3, 3) if app_ms else None,
        "quantize_GBps": round(quantize_gbps, 2),
        "quantize_prefill_us": round(float(np.median(qz_ms)) * 1e3, 2),
        "prefill_tokens": prefill_tokens,
        "quantize_layers_per_call": model_layers,
        "roofline": {"bound": "hbm", "achieved": round(dec_gbps, 2), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(dec_gbps / HBM_PEAK_GBPS, 4),
                     "traffic": measured_traffic(w.name + (f"_window{args.window}_sinks{args.sinks}"
                                                           if args.window or args.sinks else "")
                                                 + (f"_rope{args.rope_base:g}" if args.rope_base else "")),
                     "kernel": ("kvq_decode_attention_layers" if multi else
                                "kvq_decode_step (append + decode attention)" if fused_step else "kvq_decode_attention"),
                     "bytes_per_launch": int(np.mean(ev_bytes)),
                     "measured_ceiling": {"kernel": "kvq_read_probe", "bytes": probe_bytes,
                                          "GBps": round(ceiling_gbps, 2),
                                          "frac_of_peak": round(ceiling_gbps / HBM_PEAK_GBPS, 4),
                                          "decode_frac_of_ceiling": round(dec_gbps / ceiling_gbps, 4)}},
    }
    if cpu is not None:
        result["cpu_baseline"] = cpu
    print(json.dumps(result), flush=True)


def append_head_bytes(L, n, D, w, bk, bv, ib):
    """Bytes an append of n tokens to one (seq, kv head) at length L must move:
    the new rows read; channel-axis tensors: the residual rows a completed block
    reads back, the codes and (step, zero) pairs of completed blocks and the new
    rows that stay in the residual written; token-axis tensors: codes and pairs
    of every new row written."""
    tot = 0
    for axis, G, B in ((w.axis_k, w.group_k, bk), (w.axis_v, w.group_v, bv)):
        tot += n * D * ib
        if axis == 0:
            nb = (L + n) // G - L // G
            if nb:
                tot += (L % G) * D * ib + nb * (G * D * B // 8 + 4 * D) + ((L + n) % G) * D * ib
            else:
                tot += n * D * ib
        else:
            tot += n * (D * B // 8 + 4 * (D // G))
    return tot


def kernel_source_hash(sources=None):
    """Hash of the named library sources (all of them when None); a counter
    summary taken on other sources is stale."""
    import hashlib
    h = hashlib.sha256()
    csrc = os.path.join(ROOT, "bit_kv_cache_groupwise_amd", "csrc")
    names = sorted(os.listdir(csrc)) if sources is None else sorted(sources)
    for name in names:
        if name.endswith((".hip", ".h", ".cpp")):
            with open(os.path.join(csrc, name), "rb") as f:
                h.update(name.encode() + f.read())
    return h.hexdigest()[:16]


def measured_traffic(workload):
    """HBM bytes per decode launch from the committed counter summary
    (profiles/traffic_<workload>.json, <workload>_window<R>_sinks<S> with a
    full-precision window: FETCH_SIZE and WRITE_SIZE of the decode
    kernel, each divided by the bytes-per-byte factor the same counter reads on
    a plain copy of known size), or None when absent or when any source file of
    the kernels it counted (listed in the summary) has changed since."""
    path = os.path.join(ROOT, "profiles", f"traffic_{workload}.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        t = json.load(f)
    if t.get("source_hash") != kernel_source_hash(t.get("sources")):
        return None
    return t.get("traffic_bytes_per_launch")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _oracle_units(w, seqs, budget_s, window, sinks):
    """The CPU oracle, untuned, on whole (sequence, kv head) units of one decode
    step: encode the head's history (quantize + pack + fp64 dequantize), then
    attend its query heads in fp64. Stops after budget_s seconds of oracle time.
    Returns (units, algorithmic decode bytes, quantize seconds, attention seconds).
    Inputs are drawn per sequence (not timed); one BLAS / torch thread."""
    import torch
    from threadpoolctl import threadpool_limits

    from bit_kv_cache_groupwise_amd import workloads as W
    from oracle import kvq_oracle as o

    torch.set_num_threads(1)
    ib = 4 if w.in_dtype == "f32" else 2
    R = w.q_heads // w.kv_heads
    units = done = 0
    tq = ta = 0.0
    with threadpool_limits(limits=1):
        for s in seqs:
            if tq + ta >= budget_s:
                break
            T = w.lengths[s] + w.new_tokens
            bk, bv = w.bits[s]
            counts = [0] * w.num_seqs
            counts[s] = T
            k, v = W.draw_kv(w, 0, counts, stream=0)
            q = W.draw_q(w, 0)[s].double().numpy()
            k = k.float().numpy()
            v = v.float().numpy()
            kw = dict(group_k=w.group_k, group_v=w.group_v, axis_k=w.axis_k, axis_v=w.axis_v, bits_k=bk, bits_v=bv)
            for h in range(w.kv_heads):
                t0 = time.perf_counter()
                if window or sinks:
                    e = o.encode_head_window(k[:, h], v[:, h], window=window, sinks=sinks, **kw)
                else:
                    e = o.encode_head(k[:, h], v[:, h], **kw)
                t1 = time.perf_counter()
                o.attend(q[h * R:(h + 1) * R], e["k_hat"], e["v_hat"], w.softmax_scale)
                t2 = time.perf_counter()
                tq += t1 - t0
                ta += t2 - t1
                done += algorithmic_head_bytes(T, w.head_dim, w.axis_k, w.axis_v, w.group_k, w.group_v, bk, bv, ib,
                                               window, sinks)
                units += 1
                if tq + ta >= budget_s:
                    break
    return units, done, tq, ta


def _oracle_worker(a):
    return _oracle_units(*a)


def cpu_baseline(w, budget_s, window=0, sinks=0, workers=0):
    """The CPU oracle as it stands, timed on the host: on one core for about
    budget_s seconds, and on all allowed cores (forked worker processes, one
    thread each, sequences dealt round-robin) for about budget_s seconds each.
    The rate is the same algorithmic decode bytes per second as the GPU figure;
    quantize (encode) and attention seconds are reported apart."""
    import multiprocessing as mp
    from concurrent.futures import ProcessPoolExecutor

    import numpy as np

    order = [int(x) for x in np.random.Generator(np.random.PCG64(7)).permutation(w.num_seqs)]
    try:
        allowed = len(os.sched_getaffinity(0))
    except AttributeError:
        allowed = os.cpu_count() or 1
    nw = workers or max(1, min(allowed, 16))
    # all cores first: the pool forks before this process has run any threaded work
    t0 = time.perf_counter()
    with ProcessPoolExecutor(max_workers=nw, mp_context=mp.get_context("fork")) as ex:
        parts = list(ex.map(_oracle_worker, [(w, order[i::nw], budget_s, window, sinks) for i in range(nw)]))
    wall = time.perf_counter() - t0
    mu = sum(p[0] for p in parts)
    mb = sum(p[1] for p in parts)
    mq = sum(p[2] for p in parts)
    ma = sum(p[3] for p in parts)
    u1, b1, q1, a1 = _oracle_units(w, order, budget_s, window, sinks)
    total_units = w.num_seqs * w.kv_heads
    return {"value": round(mb / wall / 1e9, 6), "unit": "GB/s", "cores": nw, "kind": "oracle",
            "sample": f"{mu} of the {total_units} (seq, kv head) units of one {w.name} decode step"
                      f"{' (the whole step)' if mu == total_units else ''} on {nw} worker processes (1 thread each), "
                      f"{u1} units on one core: quantize + pack + fp64 dequantize, fp64 attention",
            "seconds": round(wall, 2),
            "cpu_model": _cpu_model(), "nproc": os.cpu_count(), "allowed_cpus": allowed,
            "all_cores": {"GBps": round(mb / wall / 1e9, 6), "units": mu, "wall_s": round(wall, 2),
                          "quantize_s_per_unit": round(mq / max(mu, 1), 4),
                          "attention_s_per_unit": round(ma / max(mu, 1), 4)},
            "single_core": {"GBps": round(b1 / max(q1 + a1, 1e-9) / 1e9, 6), "units": u1,
                            "quantize_s": round(q1, 2), "attention_s": round(a1, 2),
                            "quantize_s_per_unit": round(q1 / max(u1, 1), 4),
                            "attention_s_per_unit": round(a1 / max(u1, 1), 4)}}


if __name__ == "__main__":
    main()
