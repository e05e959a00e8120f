"""Checks that pin the CPU oracle to facts fixed outside itself: hand-derived
worked examples, exact rational arithmetic on exhaustive tiny inputs, closed
forms, library routines and the figures the pages print.

Each check takes the oracle module as an argument so that
test_oracle_mutations.py can run the same checks against deliberately broken
copies and confirm that every plausible slip fails at least one of them.
"""

from __future__ import annotations

import itertools
import math
import os
import struct
from fractions import Fraction

import numpy as np

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _read_kv(path):
    out = {}
    with open(path) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            key, *vals = line.split()
            out[key] = vals
    return out


def round_half_even(fr: Fraction) -> int:
    fl = math.floor(fr)
    rem = fr - fl
    if rem > Fraction(1, 2):
        return fl + 1
    if rem < Fraction(1, 2):
        return fl
    return fl if fl % 2 == 0 else fl + 1


def f16_bits(x: float) -> int:
    """float -> fp16 bit pattern via the struct module (IEEE binary16, nearest-even)."""
    return struct.unpack("<H", struct.pack("<e", x))[0]


# ----------------------------------------------------------------------------
# Quantizer
# ----------------------------------------------------------------------------

def check_worked_example(o):
    g = _read_kv(os.path.join(GOLDEN, "rne_worked_example.txt"))
    bits = int(g["bits"][0])
    x = np.array([float(v) for v in g["values"]], np.float32)
    s, z = o.group_params(x.min(), x.max(), bits)
    assert float(s) == float(g["step"][0]), (s, g["step"])
    assert float(z) == float(g["zero"][0]), (z, g["zero"])
    codes = o.encode_values(x, s, z, bits)
    assert codes.tolist() == [int(c) for c in g["codes"]], codes


def check_brute_force_nearest(o, bits_list=(2, 3), max_group=4):
    """Exhaustive tiny groups: every code is the nearest level of the stored grid
    computed in exact rational arithmetic (ties to even), except within 2^-18
    of a midpoint, where float32 rounding of t may pick either neighbour."""
    grid = [-2.0, -1.0, -0.75, -0.5, 0.0, 0.1, 0.25, 0.5, 1.0, 1.5, 3.0]
    checked = 0
    for bits in bits_list:
        L = (1 << bits) - 1
        for n in range(2, max_group + 1):
            for combo in itertools.product(grid, repeat=n):
                x = np.array(combo, np.float32)
                mn, mx = Fraction(float(x.min())), Fraction(float(x.max()))
                s, z = o.group_params(x.min(), x.max(), bits)
                # stored step and zero are the fp16 roundings of the exact definitions
                s_exact32 = np.float32(np.float32(x.max()) - np.float32(x.min())) / np.float32(L)
                assert f16_bits(float(s)) == f16_bits(float(s_exact32)), (combo, bits)
                assert f16_bits(float(z)) == f16_bits(float(mn)), (combo, bits)
                assert abs(Fraction(float(s)) - (mx - mn) / L) <= (mx - mn) / L * Fraction(1, 1024) + Fraction(1, 2**24)
                codes = o.encode_values(x, s, z, bits)
                S, Z = Fraction(float(s)), Fraction(float(z))
                for xi, ci in zip(combo, codes.tolist()):
                    if S == 0:
                        assert ci == 0
                        continue
                    t = (Fraction(xi) - Z) / S
                    want = min(max(round_half_even(t), 0), L)
                    if ci != want:
                        near = abs((t - math.floor(t)) - Fraction(1, 2)) <= Fraction(1, 2**18) * max(1, abs(t))
                        assert near and abs(ci - want) == 1, (combo, bits, xi, ci, want, float(t))
                    checked += 1
    assert checked > 10000


def _random_groups(rng, n_groups, G):
    kinds = []
    for i in range(n_groups):
        k = i % 4
        if k == 0:
            g = rng.standard_normal(G)
        elif k == 1:
            g = rng.standard_normal(G) * 0.01 + 3.0
        elif k == 2:
            g = rng.standard_normal(G)
            g[rng.integers(G)] *= 100.0  # one outlier inflates the step
        else:
            g = rng.uniform(-1000, 1000, G)
        kinds.append(g)
    return np.array(kinds, np.float16).astype(np.float32)  # fp16-representable inputs


def check_half_step_bound(o, seed=0):
    """|x - x_hat| <= step/2 for every element whose rounded t is in range
    ([U] "O Que o Erro ...": the error is bounded by half a step)."""
    rng = np.random.default_rng(seed)
    for bits in (2, 3, 4, 6, 8):
        xg = _random_groups(rng, 400, 32)
        s, z = o.group_params(xg.min(axis=1), xg.max(axis=1), bits)
        codes = o.encode_values(xg, s[:, None], z[:, None], bits)
        xhat = z[:, None].astype(np.float64) + codes.astype(np.float64) * s[:, None].astype(np.float64)
        t = (xg.astype(np.float64) - z[:, None]) / np.where(s == 0, 1, s)[:, None]
        unclamped = (np.rint(t) >= 0) & (np.rint(t) <= (1 << bits) - 1)
        err = np.abs(xg.astype(np.float64) - xhat)
        bound = s[:, None].astype(np.float64) / 2 * (1 + 2.0**-18)
        assert np.all(err[unclamped] <= np.broadcast_to(bound, err.shape)[unclamped]), bits
        assert unclamped.mean() > 0.9


def check_min_max_codes(o, seed=1):
    """The group minimum maps to code 0 and the maximum to 2^B - 1."""
    rng = np.random.default_rng(seed)
    for bits in (2, 3, 4, 6, 8):
        xg = _random_groups(rng, 200, 32)
        s, z = o.group_params(xg.min(axis=1), xg.max(axis=1), bits)
        codes = o.encode_values(xg, s[:, None], z[:, None], bits)
        imin = xg.argmin(axis=1)
        imax = xg.argmax(axis=1)
        r = np.arange(len(xg))
        assert np.all(codes[r, imin] == 0)
        assert np.all(codes[r, imax] == (1 << bits) - 1)


def check_monotone(o, seed=2):
    rng = np.random.default_rng(seed)
    for bits in (2, 3, 4, 6, 8):
        xg = _random_groups(rng, 100, 64)
        s, z = o.group_params(xg.min(axis=1), xg.max(axis=1), bits)
        codes = o.encode_values(xg, s[:, None], z[:, None], bits).astype(int)
        order = np.argsort(xg, axis=1, kind="stable")
        srt = np.take_along_axis(codes, order, axis=1)
        assert np.all(np.diff(srt, axis=1) >= 0)


def check_exact_reconstruction(o):
    """When the step (max - min)/(2^B - 1) is exactly representable, the group
    minimum, maximum and every grid point z + k*s reconstruct exactly."""
    rng = np.random.default_rng(3)
    for bits in (2, 3, 4, 6, 8):
        L = (1 << bits) - 1
        for _ in range(50):
            step = 2.0 ** int(rng.integers(-6, 3))
            zero = step * int(rng.integers(-64, 65))  # on the grid, so every x is exact in fp16
            k = rng.integers(0, L + 1, 32)
            k[0], k[1] = 0, L
            x = (zero + k * step).astype(np.float32)
            codes, s, z, resid = o.quantize_tensor(x[None, :], o.AXIS_TOKEN, 32, bits)
            xhat = o.dequantize_tensor(codes, s, z, resid, o.AXIS_TOKEN, 32)[0]
            assert float(s[0, 0]) == step and float(z[0, 0]) == zero
            assert np.array_equal(codes[0], k.astype(np.uint8))
            assert np.array_equal(xhat, x.astype(np.float64))
            assert xhat.min() == x.min() and xhat.max() == x.max()


def check_b8_bound(o, seed=4):
    """At 8 bits the error is at most range/510, up to the rounding of the stored
    step and zero to fp16."""
    rng = np.random.default_rng(seed)
    xg = _random_groups(rng, 400, 32)
    s, z = o.group_params(xg.min(axis=1), xg.max(axis=1), 8)
    codes = o.encode_values(xg, s[:, None], z[:, None], 8)
    xhat = z[:, None].astype(np.float64) + codes * s[:, None].astype(np.float64)
    rng_ = (xg.max(axis=1) - xg.min(axis=1)).astype(np.float64)
    bound = rng_ / 510 * (1 + 2.0**-9) + np.abs(xg.min(axis=1) - z) + 255 * np.abs(s - rng_ / 255)
    err = np.abs(xg - xhat).max(axis=1)
    assert np.all(err <= bound + 1e-12)


def check_constant_group(o):
    for bits in (2, 3, 4, 6, 8):
        x = np.full(32, 0.3, np.float32)
        s, z = o.group_params(x.min(), x.max(), bits)
        assert float(s) == 0.0
        assert float(z) == float(np.float16(0.3))
        assert np.all(o.encode_values(x, s, z, bits) == 0)


def check_meta_rounding(o):
    """Stored metadata equals the IEEE binary16 nearest-even rounding from the
    struct module, including exact ties and subnormals."""
    vals = [0.1, 1.0 + 2.0**-11, 1.0 + 3 * 2.0**-11, 2.0**-25, 3 * 2.0**-26, 65504.0, -7.3, 1e-7, 2.0**-24 * 1.5]
    rng = np.random.default_rng(5)
    vals += list(rng.standard_normal(500) * 10.0 ** rng.uniform(-6, 4, 500))
    got = o.to_meta(np.array(vals, np.float32))
    for v, g in zip(vals, got):
        v32 = float(np.float32(v))
        assert f16_bits(float(g)) == f16_bits(v32), (v, g)
        assert float(g) == struct.unpack("<e", struct.pack("<e", v32))[0]


def check_axis_semantics(o):
    """Keys with fixed outlier channels: per-channel groups give a smaller key
    reconstruction error than per-token groups ([U] "Chaves ...": grouping along
    tokens lets the outlier channels set every group's step)."""
    rng = np.random.default_rng(6)
    T, D = 256, 64
    m = np.ones(D)
    m[[5, 40]] = 30.0
    k = (rng.standard_normal((T, D)) * m).astype(np.float32)
    for bits in (2, 4):
        per_ch = o.quantize_tensor(k, o.AXIS_CHANNEL, 32, bits)
        per_tok = o.quantize_tensor(k, o.AXIS_TOKEN, 32, bits)
        e_ch = np.abs(o.dequantize_tensor(*per_ch, o.AXIS_CHANNEL, 32) - k).mean()
        e_tok = np.abs(o.dequantize_tensor(*per_tok, o.AXIS_TOKEN, 32) - k).mean()
        assert e_ch < 0.5 * e_tok, (bits, e_ch, e_tok)
    # and the channel-axis statistics really run over tokens: a key block whose
    # channel c is constant over its 32 tokens has step 0 in that channel only
    k2 = rng.standard_normal((64, D)).astype(np.float32)
    k2[:32, 7] = 1.25
    codes, s, z, resid = o.quantize_tensor(k2, o.AXIS_CHANNEL, 32, 2)
    assert s.shape == (2, D) and float(s[0, 7]) == 0.0 and np.all(s[0, :7] > 0) and float(s[1, 7]) > 0
    assert resid.shape == (0, D)
    codes, s, z, resid = o.quantize_tensor(k2[:50], o.AXIS_CHANNEL, 32, 2)
    assert codes.shape == (32, D) and np.array_equal(resid, k2[32:50])
    # token axis: a token whose first 32 channels are constant has step 0 in group 0 only
    k3 = rng.standard_normal((4, D)).astype(np.float32)
    k3[2, :32] = -0.5
    codes, s, z, resid = o.quantize_tensor(k3, o.AXIS_TOKEN, 32, 2)
    assert s.shape == (4, 2) and float(s[2, 0]) == 0.0 and float(s[2, 1]) > 0 and np.all(s[[0, 1, 3]] > 0)


def check_dequant_exact(o, seed=7):
    """float64 reconstruction equals z + code*s in exact rational arithmetic."""
    rng = np.random.default_rng(seed)
    x = (rng.standard_normal((64, 64)) * 5).astype(np.float32)
    for axis in (o.AXIS_CHANNEL, o.AXIS_TOKEN):
        for bits in (2, 3, 8):
            codes, s, z, resid = o.quantize_tensor(x, axis, 32, bits)
            xhat = o.dequantize_tensor(codes, s, z, resid, axis, 32)
            for _ in range(200):
                t, c = int(rng.integers(64)), int(rng.integers(64))
                if axis == o.AXIS_CHANNEL:
                    S, Z = s[t // 32, c], z[t // 32, c]
                else:
                    S, Z = s[t, c // 32], z[t, c // 32]
                exact = Fraction(float(Z)) + int(codes[t, c]) * Fraction(float(S))
                assert Fraction(float(xhat[t, c])) == exact


# ----------------------------------------------------------------------------
# Storage format
# ----------------------------------------------------------------------------

def check_pack_golden(o):
    words = {}
    with open(os.path.join(GOLDEN, "pack_words.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                b, *ws = line.split()
                words[int(b)] = [int(w, 16) for w in ws]
    assert sorted(words) == [2, 3, 4, 6, 8]
    for bits, want in words.items():
        codes = (np.arange(32) % (1 << bits)).astype(np.uint8)[None, :]
        got = o.pack_rows(codes, bits)[0].tolist()
        assert got == want, (bits, [hex(w) for w in got])


def check_pack_bigint(o, seed=8):
    """pack_rows equals the bitstream built with Python integers, unit by unit,
    and unpack_rows inverts it."""
    rng = np.random.default_rng(seed)
    for bits in (2, 3, 4, 6, 8):
        for D in (32, 64, 128, 256):
            codes = rng.integers(0, 1 << bits, (5, D)).astype(np.uint8)
            w = o.pack_rows(codes, bits)
            assert w.shape == (5, D * bits // 32) and w.dtype == np.uint32
            for r in range(5):
                for u in range(D // 32):
                    stream = 0
                    for j in range(32):
                        stream |= int(codes[r, 32 * u + j]) << (j * bits)
                    for k in range(bits):
                        assert int(w[r, u * bits + k]) == (stream >> (32 * k)) & 0xFFFFFFFF
            assert np.array_equal(o.unpack_rows(w, bits, D), codes)


def check_meta_words(o):
    s = np.array([1.0, 0.5], np.float32)
    z = np.array([-1.0, 2.0], np.float32)
    w = o.meta_words(s, z)
    # fp16 1.0 = 0x3c00, -1.0 = 0xbc00, 0.5 = 0x3800, 2.0 = 0x4000
    assert w.tolist() == [0xBC003C00, 0x40003800]


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def _python_attention(q, K, V, scale):
    """Pure-Python softmax attention for tiny inputs."""
    logits = [scale * sum(a * b for a, b in zip(q, k)) for k in K]
    m = max(logits)
    w = [math.exp(l - m) for l in logits]
    tot = sum(w)
    return [sum(wi * v[c] for wi, v in zip(w, V)) / tot for c in range(len(V[0]))]


def check_attention_closed_forms(o, seed=9):
    rng = np.random.default_rng(seed)
    T, D = 50, 32
    K = rng.standard_normal((T, D))
    V = rng.standard_normal((T, D))
    # q = 0: uniform weights -> mean of V
    out = o.attend(np.zeros((1, D)), K, V, 0.2)
    assert np.allclose(out[0], V.mean(axis=0), rtol=0, atol=1e-13)
    # one token: its value
    out = o.attend(rng.standard_normal((2, D)), K[:1], V[:1], 0.2)
    assert np.allclose(out, V[:1].repeat(2, 0), rtol=0, atol=1e-14)
    # all keys equal: mean of V
    out = o.attend(rng.standard_normal((1, D)), np.tile(K[:1], (T, 1)), V, 0.2)
    assert np.allclose(out[0], V.mean(axis=0), rtol=0, atol=1e-13)
    # one key dominates: its value
    K2 = K.copy()
    q = rng.standard_normal(D)
    K2[17] = 1000 * q
    out = o.attend(q[None], K2, V, 1.0)
    assert np.allclose(out[0], V[17], atol=1e-12)
    # brute force in pure Python
    q = rng.standard_normal((3, D))
    out = o.attend(q, K[:9], V[:9], 0.7)
    for r in range(3):
        ref = _python_attention(list(q[r]), K[:9].tolist(), V[:9].tolist(), 0.7)
        assert np.allclose(out[r], ref, rtol=1e-12, atol=1e-14)
    # empty history
    assert np.all(o.attend(q, K[:0], V[:0], 1.0) == 0)
    # grouped-query map: query head h reads kv head h // (Hq/Hkv)
    Kh = rng.standard_normal((2, 7, D))
    Vh = rng.standard_normal((2, 7, D))
    qh = rng.standard_normal((6, D))
    out = o.attend_heads(qh, Kh, Vh, 0.3)
    for h in range(6):
        ref = _python_attention(list(qh[h]), Kh[h // 3].tolist(), Vh[h // 3].tolist(), 0.3)
        assert np.allclose(out[h], ref, rtol=1e-12, atol=1e-14)


def check_attention_vs_torch(o, seed=10):
    """An all-residual key cache (fewer than G tokens) with 8-bit values against
    torch's scaled_dot_product_attention in float64."""
    import torch
    rng = np.random.default_rng(seed)
    T, D = 20, 64
    k = rng.standard_normal((T, D)).astype(np.float32)
    v = rng.standard_normal((T, D)).astype(np.float32)
    enc = o.encode_head(k, v, group_k=32, group_v=32, axis_k=o.AXIS_CHANNEL, axis_v=o.AXIS_TOKEN,
                        bits_k=8, bits_v=8)
    assert enc["k_codes"].shape == (0, D) and np.array_equal(enc["k_hat"], k.astype(np.float64))
    q = rng.standard_normal((4, D))
    out = o.attend(q, enc["k_hat"], enc["v_hat"], 1 / 8)
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(enc["k_hat"])[None, None].expand(1, 4, T, D),
        torch.from_numpy(enc["v_hat"])[None, None].expand(1, 4, T, D), scale=1 / 8)[0, :, 0, :].numpy()
    assert np.allclose(out, ref, rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------
# Sizes
# ----------------------------------------------------------------------------

def check_sizes(o):
    """Bytes per (layer, sequence, kv head) against the closed form, and the
    cache-element formula ([N] "Ukuran cache bertambah ...")."""
    assert o.cache_elements(32, 4096, 32, 128) == 2 * 32 * 4096 * 32 * 128
    # 8-bit K and V with no metadata: bytes = elements
    b = o.head_bytes(4096, 128, group_k=32, group_v=32, axis_k=o.AXIS_TOKEN, axis_v=o.AXIS_TOKEN,
                     bits_k=8, bits_v=8, in_bytes=2, meta_bytes=0)
    assert b["total"] == o.cache_elements(1, 4096, 1, 128)  # 8-bit codes: one byte per element
    for T in (0, 1, 31, 32, 33, 4097):
        for (bk, bv) in ((2, 2), (3, 3), (4, 4), (6, 4), (4, 8)):
            b = o.head_bytes(T, 128, group_k=32, group_v=32, axis_k=o.AXIS_CHANNEL, axis_v=o.AXIS_TOKEN,
                             bits_k=bk, bits_v=bv, in_bytes=2)
            tq = T - T % 32
            assert b["codes"] == tq * 128 * bk // 8 + T * 128 * bv // 8
            assert b["meta"] == 4 * (tq // 32) * 128 + 4 * T * 4
            assert b["residual"] == (T % 32) * 128 * 2
            assert b["total"] == b["codes"] + b["meta"] + b["residual"]


def check_sizing_pages(o):
    """Effective bits and compression ratios printed on hatterialabs.com,
    "Asymetrie kvantizace KV cache"."""
    figs = {}
    with open(os.path.join(GOLDEN, "sizing_pages.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                name, _, val, _ = [p.strip() for p in line.split("|")]
                figs[name] = float(val)
    # GPT-2 small: K6/V4, per-head groups of 64 channels
    eb = o.effective_bits(6, 4, 64, 64)
    assert eb == figs["gpt2_k6v4_effective_bits"]
    assert round(16 / eb, 1) == figs["gpt2_k6v4_ratio"]
    # and the same figure from our byte accounting of a GPT-2-shaped head (64
    # channels; K per-channel over 64-token blocks, V per-token over the head)
    T = 1024
    hb = o.head_bytes(T, 64, group_k=64, group_v=64, axis_k=o.AXIS_CHANNEL, axis_v=o.AXIS_TOKEN,
                      bits_k=6, bits_v=4, in_bytes=2)
    assert hb["total"] * 8 / (2 * T * 64) == figs["gpt2_k6v4_effective_bits"]
    assert round(16 / 6.5, 1) == figs["knee_ratio_low"]
    # K4/V8 with head_dim 256 per-head groups against bf16
    eb = o.effective_bits(4, 8, 256, 256)
    assert round(16 / eb, 1) == figs["qwen_k4v8_ratio"]
    assert round(8.6 * (1 - eb / 16), 1) == figs["qwen_k4v8_saved_gb"]


# ----------------------------------------------------------------------------
# Full-precision recent window and sinks ([U] "O Imposto dos Sistemas ...",
# "O Que Fazer Com Isso", "Onde o Trabalho Esta Indo")
# ----------------------------------------------------------------------------

def check_window_blocks(o):
    """The quantized tokens under a window of R and S sinks are exactly the
    union of the whole key blocks inside [S, len - R), enumerated block by block;
    the recent full-precision part then holds between R and R + Gb - 1 tokens."""
    for block in (1, 32, 64):
        for sinks in (0, block, 2 * block) if block > 1 else (0, 1, 4):
            for window in (0, 1, 31, 32, 100, 128):
                if window == 0 and sinks == 0:
                    continue
                for length in list(range(0, 300, 7)) + [sinks + window + block, 1000, 1023, 1024, 1025]:
                    quant = np.zeros(length, dtype=bool)
                    b = 0
                    while (b + 1) * block <= length:
                        lo, hi = b * block, (b + 1) * block
                        if lo >= sinks and hi <= length - window:
                            quant[lo:hi] = True
                        b += 1
                    got = o.full_precision_mask(length, window, sinks, block)
                    assert got.shape == (length,) and got.dtype == bool
                    assert np.array_equal(~got, quant), (block, sinks, window, length)
                    if length >= sinks + window:
                        recent = int(got[sinks:].sum())
                        assert window <= recent <= window + block - 1, (block, sinks, window, length, recent)
    # no window: nothing beyond the residual of R4
    assert not o.full_precision_mask(100, 0, 0, 32).any()
    assert o.token_block(o.AXIS_CHANNEL, 64, o.AXIS_TOKEN, 32) == 64
    assert o.token_block(o.AXIS_TOKEN, 64, o.AXIS_TOKEN, 32) == 1


def check_window_exact_attention(o, seed=11):
    """A window at least as long as the cache (or sinks covering it) makes the
    attention exact: torch's scaled_dot_product_attention in float64 over the
    unquantized rows. A partial window keeps the stored bytes of the plain
    encoding, takes exact rows where the mask is set and the plain
    reconstruction elsewhere."""
    import torch
    rng = np.random.default_rng(seed)
    T, D = 100, 64
    k = (rng.standard_normal((T, D)) * rng.uniform(0.5, 8, D)).astype(np.float32)
    v = rng.standard_normal((T, D)).astype(np.float32)
    q = rng.standard_normal((2, D))
    ref = torch.nn.functional.scaled_dot_product_attention(
        torch.from_numpy(q)[None, :, None, :], torch.from_numpy(k.astype(np.float64))[None, None].expand(1, 2, T, D),
        torch.from_numpy(v.astype(np.float64))[None, None].expand(1, 2, T, D), scale=0.125)[0, :, 0, :].numpy()
    kw = dict(group_k=32, group_v=32, axis_k=o.AXIS_CHANNEL, axis_v=o.AXIS_TOKEN, bits_k=2, bits_v=2)
    for window, sinks in ((T, 0), (T + 5, 32), (0, 128), (200, 96)):
        enc = o.encode_head_window(k, v, window=window, sinks=sinks, **kw)
        assert np.array_equal(enc["k_hat"], k.astype(np.float64)) and np.array_equal(enc["v_hat"], v.astype(np.float64))
        assert np.allclose(o.attend(q, enc["k_hat"], enc["v_hat"], 0.125), ref, rtol=1e-12, atol=1e-13)
    plain = o.encode_head(k, v, **kw)
    enc = o.encode_head_window(k, v, window=20, sinks=32, **kw)
    for name in ("k_words", "v_words", "k_meta", "v_meta", "k_resid"):
        assert np.array_equal(enc[name], plain[name]), name
    m = enc["fp_mask"]
    # sinks [0, 32); block [32, 64) ends before 100 - 20 = 80; block [64, 96) does not
    assert np.array_equal(np.nonzero(~m)[0], np.arange(32, 64))
    for x, hat, ph in ((k, enc["k_hat"], plain["k_hat"]), (v, enc["v_hat"], plain["v_hat"])):
        assert np.array_equal(hat[m], x[m].astype(np.float64))
        assert np.array_equal(hat[~m], ph[~m])
    # the quantized part must be used: 2-bit keys move the output away from exact
    assert not np.allclose(o.attend(q, enc["k_hat"], enc["v_hat"], 0.125), ref, atol=1e-3)


# ----------------------------------------------------------------------------
# Rotary positions after dequantization ([U] "Embebedos Rotatorios Complicam
# as Chaves")
# ----------------------------------------------------------------------------

def check_rope_complex_form(o, seed=12):
    """The rotation equals complex multiplication: channel pair (i, i + D/2) as
    a + jb times e^(j t theta_i); frequencies from the golden values (base
    10000, D = 8: 1, 0.1, 0.01, 0.001); position 0 is the identity; norms and
    relative positions are preserved."""
    g = _read_kv(os.path.join(GOLDEN, "rope_frequencies.txt"))
    th = o.rope_frequencies(int(g["head_dim"][0]), float(g["base"][0]))
    np.testing.assert_allclose(th, [float(v) for v in g["theta"]], rtol=1e-15)
    rng = np.random.default_rng(seed)
    D, T = 64, 50
    x = rng.standard_normal((T, D))
    pos = rng.integers(0, 300000, T)
    got = o.rope(x, pos, 10000.0)
    z = (x[:, :D // 2] + 1j * x[:, D // 2:]) * np.exp(1j * np.outer(pos, o.rope_frequencies(D, 10000.0)))
    np.testing.assert_allclose(got, np.concatenate([z.real, z.imag], axis=1), rtol=1e-9, atol=1e-9)
    np.testing.assert_array_equal(o.rope(x, np.zeros(T, int), 10000.0), x)
    np.testing.assert_allclose(np.linalg.norm(got, axis=1), np.linalg.norm(x, axis=1), rtol=1e-12)
    q, k = rng.standard_normal((1, D)), rng.standard_normal((1, D))
    d0 = float((o.rope(q, [17], 500.0) @ o.rope(k, [5], 500.0).T)[0, 0])
    d1 = float((o.rope(q, [1017], 500.0) @ o.rope(k, [1005], 500.0).T)[0, 0])
    assert abs(d0 - d1) < 1e-9 * max(1.0, abs(d0))


def check_rope_attention(o, seed=13):
    """attend_rope scores q against the key rotated to its own position: a single
    key rotated by hand (2 x 2 rotations), and position-0 rotation being the plain
    attention."""
    rng = np.random.default_rng(seed)
    D = 4
    k = np.array([[1.0, 2.0, 3.0, 4.0], [0.5, -1.0, 0.0, 2.0]])
    v = rng.standard_normal((2, D))
    q = rng.standard_normal((1, D))
    th = [1.0, 0.01]  # base 10000, D = 4
    k1 = k[1]
    k1r = np.array([k1[0] * math.cos(th[0]) - k1[2] * math.sin(th[0]), k1[1] * math.cos(th[1]) - k1[3] * math.sin(th[1]),
                    k1[0] * math.sin(th[0]) + k1[2] * math.cos(th[0]), k1[1] * math.sin(th[1]) + k1[3] * math.cos(th[1])])
    lg = np.array([q[0] @ k[0], q[0] @ k1r]) * 0.5
    w = np.exp(lg - lg.max())
    w /= w.sum()
    np.testing.assert_allclose(o.attend_rope(q, k, v, 0.5, 10000.0)[0], w @ v, rtol=1e-12)
    np.testing.assert_allclose(o.attend_rope(q, k[:1], v[:1], 0.5, 10000.0), o.attend(q, k[:1], v[:1], 0.5))



# ----------------------------------------------------------------------------
# Adversarial groups, in exact rational arithmetic
# ----------------------------------------------------------------------------

def round_to_format(fr: Fraction, frac_bits: int, emin: int) -> Fraction:
    """Nearest value (ties to even) of a binary floating-point format with
    ``frac_bits`` fraction bits and smallest normal exponent ``emin``
    (subnormals included; no overflow in the inputs used here)."""
    if fr == 0:
        return Fraction(0)
    sign = -1 if fr < 0 else 1
    a = abs(fr)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    while Fraction(2) ** (e + 1) <= a:
        e += 1
    ulp = Fraction(2) ** (max(e, emin) - frac_bits)
    return sign * round_half_even(a / ulp) * ulp


def r32(fr):
    return round_to_format(fr, 23, -126)


def r16(fr):
    return round_to_format(fr, 10, -14)


def check_edge_groups_exact(o):
    """Constant groups, fp16-subnormal and underflowing steps, exact ties and
    near ties (t within 2^-13 of k + 1/2 but not on it), clamping after the fp16 rounding of the step or the zero, magnitudes below
    fp16's range and near 65504: step, zero, codes and reconstruction of the
    oracle equal the definition evaluated in exact rationals with every float32
    and fp16 rounding written out (zero = min, step = fp32(fp32(max - min) /
    (2^B - 1)), both stored in fp16; t = fp32(fp32(x - z) / s); code =
    clamp(round-half-even(t), 0, 2^B - 1); 0 where s = 0; x_hat = z + code*s)
    ([U] "O Que o Erro de Quantizacao ..."; [N] "Scale menentukan ...")."""
    from tests import edge_inputs as E
    seen = set()
    for dtype in ("f32", "f16", "bf16"):
        for bits in (2, 3, 4, 6, 8):
            L = (1 << bits) - 1
            for name, g in E.groups(bits, dtype, seed=5):
                xs = [Fraction(float(v)) for v in g]
                mn, mx = min(xs), max(xs)
                s = r16(r32(r32(mx - mn) / L))
                z = r16(mn)
                want = []
                for x in xs:
                    if s == 0:
                        want.append(0)
                    else:
                        t = r32(r32(x - z) / s)
                        want.append(min(max(round_half_even(t), 0), L))
                gs, gz = o.group_params(g.min(), g.max(), bits)
                assert Fraction(float(gs)) == s and Fraction(float(gz)) == z, (dtype, bits, name, gs, gz, s, z)
                codes = o.encode_values(g, gs, gz, bits)
                assert [int(c) for c in codes] == want, (dtype, bits, name)
                xq = o.dequantize_tensor(codes[:, None], np.array([[gs]]), np.array([[gz]]), np.zeros((0, 1)),
                                         o.AXIS_CHANNEL, len(g))
                for c, v in zip(want, xq[:, 0]):
                    assert Fraction(float(v)) == z + c * s, (dtype, bits, name)
                seen.add(name.split("_")[0])
                if name.startswith("substep") and L + 1 <= int(name.split("_")[1]) <= 2 * L - 1:
                    seen.add("clamp_top" if max(want) == L and any(
                        round_half_even(r32(r32(x - z) / s)) > L for x in xs) else "noclamp")
                if name.startswith("zero_rounds_up"):
                    seen.add("zero_above_min" if z > mn else "zero_below")
                if s == 0 and mx > mn:
                    seen.add("step_underflow")
                if name.startswith("neartie") and s != 0 and any(
                        0 < abs(abs(r32(r32(x - z) / s) - round_half_even(r32(r32(x - z) / s))) - Fraction(1, 2))
                        < Fraction(1, 2 ** 13) for x in xs):
                    seen.add("near_tie_band")
    # the cases exercise what they are named for
    for need in ("const", "ties", "neartie", "substep", "underflow", "tiny", "big", "clamp_top", "zero_above_min",
                 "step_underflow", "near_tie_band"):
        assert need in seen, need


ALL_CHECKS = [
    check_worked_example, check_brute_force_nearest, check_half_step_bound, check_min_max_codes,
    check_monotone, check_exact_reconstruction, check_b8_bound, check_constant_group,
    check_meta_rounding, check_axis_semantics, check_dequant_exact, check_pack_golden,
    check_pack_bigint, check_meta_words, check_attention_closed_forms, check_attention_vs_torch,
    check_sizes, check_sizing_pages, check_window_blocks, check_window_exact_attention,
    check_rope_complex_form, check_rope_attention, check_edge_groups_exact,
]
