"""Plant plausible mistakes in copies of the oracle (on the CPU) and check that
at least one pin catches each of them."""

import importlib.util
import os

import numpy as np
import pytest

from tests import oracle_pins

ORACLE_SRC = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle", "kvq_oracle.py")


def fresh_oracle():
    spec = importlib.util.spec_from_file_location("kvq_oracle_mutant", ORACLE_SRC)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def m_levels_pow2(o):
    o.levels = lambda bits: 1 << bits


def m_round_half_up(o):
    orig = o.encode_values

    def enc(x, s, z, bits):
        x = np.asarray(x, np.float32); s = np.asarray(s, np.float32); z = np.asarray(z, np.float32)
        sd = np.where(s == 0, np.float32(1), s).astype(np.float32)
        t = (x - z) / sd
        k = np.clip(np.floor(t + np.float32(0.5)), 0, (1 << bits) - 1)
        return np.where(s == 0, 0, k).astype(np.uint8)
    o.encode_values = enc


def m_clamp_off_by_one(o):
    def enc(x, s, z, bits):
        x = np.asarray(x, np.float32); s = np.asarray(s, np.float32); z = np.asarray(z, np.float32)
        sd = np.where(s == 0, np.float32(1), s).astype(np.float32)
        k = np.clip(np.rint((x - z) / sd), 0, (1 << bits) - 2)
        return np.where(s == 0, 0, k).astype(np.uint8)
    o.encode_values = enc


def m_zero_is_max(o):
    orig = o.group_params
    o.group_params = lambda mn, mx, bits, meta_dtype="f16": orig(mx, mn, bits, meta_dtype)


def m_unrounded_grid(o):
    def gp(mn, mx, bits, meta_dtype="f16"):
        mn = np.asarray(mn, np.float32); mx = np.asarray(mx, np.float32)
        return (mx - mn) / np.float32((1 << bits) - 1), mn  # skips the fp16 rounding
    o.group_params = gp


def m_meta_truncate(o):
    def tm(v, meta_dtype="f16"):
        v = np.asarray(v, np.float32)
        b = v.view(np.uint32) & np.uint32(0xFFFFE000)  # chop the mantissa
        return b.view(np.float32).astype(np.float16).astype(np.float32)
    o.to_meta = tm


def m_axis_swapped(o):
    orig = o.quantize_tensor
    o.quantize_tensor = lambda x, axis, group, bits, meta_dtype="f16": orig(x, 1 - axis, group, bits, meta_dtype)


def m_pack_msb_first(o):
    orig = o.pack_rows

    def pack(codes, bits):
        w = orig(codes, bits)
        # reverse the bit order inside every word
        out = np.zeros_like(w)
        for i in range(32):
            out |= ((w >> np.uint32(i)) & np.uint32(1)) << np.uint32(31 - i)
        return out
    o.pack_rows = pack


def m_dequant_midrise(o):
    orig = o.dequantize_tensor

    def dq(codes, s, z, resid, axis, group):
        return orig(np.asarray(codes, np.float64) + 0.5, s, z, resid, axis, group)
    o.dequantize_tensor = dq


def m_softmax_no_scale(o):
    orig = o.attend
    o.attend = lambda q, k, v, scale: orig(q, k, v, 1.0)


def m_gqa_modulo(o):
    def ah(q, khat, vhat, scale):
        q = np.asarray(q, np.float64)
        out = np.zeros(q.shape)
        for h in range(q.shape[0]):
            out[h] = o.attend(q[h:h + 1], khat[h % len(khat)], vhat[h % len(khat)], scale)[0]
        return out
    o.attend_heads = ah


def m_weights_unnormalised(o):
    def att(q, khat, vhat, scale):
        q = np.asarray(q, np.float64)
        if len(khat) == 0:
            return np.zeros(q.shape)
        lg = scale * (q @ np.asarray(khat, np.float64).T)
        return np.exp(lg - lg.max(axis=1, keepdims=True)) @ np.asarray(vhat, np.float64)
    o.attend = att


def m_residual_dropped(o):
    orig = o.quantize_tensor

    def qt(x, axis, group, bits, meta_dtype="f16"):
        c, s, z, r = orig(x, axis, group, bits, meta_dtype)
        return c, s, z, r[:0]
    o.quantize_tensor = qt


def m_meta_bytes_halved(o):
    orig = o.head_bytes
    o.head_bytes = lambda *a, **k: orig(*a, **{**k, "meta_bytes": 2})
    orig_eb = o.effective_bits
    o.effective_bits = lambda bk, bv, gk, gv, meta_bits=32: orig_eb(bk, bv, gk, gv, 16)


def m_window_rounds_up(o):
    def fpm(length, window, sinks, block):
        t = np.arange(length)
        if window == 0 and sinks == 0:
            return np.zeros(length, dtype=bool)
        q = max(sinks, block * (-(-(length - window) // block)))  # ceiling: a block too many
        return (t < sinks) | (t >= q)
    o.full_precision_mask = fpm


def m_window_no_sinks(o):
    orig = o.full_precision_mask

    def fpm(length, window, sinks, block):
        m = orig(length, window, sinks, block)
        m[:sinks] = False if window else m[:sinks]
        return m
    o.full_precision_mask = fpm


def m_window_keys_only(o):
    orig = o.apply_window
    calls = {"n": 0}

    def aw(x, x_hat, mask):
        calls["n"] += 1
        return orig(x, x_hat, mask) if calls["n"] % 2 == 1 else np.array(x_hat, dtype=np.float64)
    o.apply_window = aw


def m_window_exact_tokens(o):
    def fpm(length, window, sinks, block):
        t = np.arange(length)
        if window == 0 and sinks == 0:
            return np.zeros(length, dtype=bool)
        return (t < sinks) | (t >= length - window)  # ignores the block boundary
    o.full_precision_mask = fpm


def m_rope_sign(o):
    orig = o.rope
    o.rope = lambda x, positions, base: orig(x, -np.asarray(positions), base)


def m_rope_interleaved(o):
    def rope(x, positions, base):
        x = np.asarray(x, dtype=np.float64)
        D = x.shape[1]
        ang = np.asarray(positions, dtype=np.float64)[:, None] * o.rope_frequencies(D, base)[None, :]
        c, s = np.cos(ang), np.sin(ang)
        a, b = x[:, 0::2], x[:, 1::2]  # pairs (2i, 2i+1) instead of (i, i + D/2)
        out = np.empty_like(x)
        out[:, 0::2] = a * c - b * s
        out[:, 1::2] = a * s + b * c
        return out
    o.rope = rope


def m_rope_freq_exponent(o):
    o.rope_frequencies = lambda head_dim, base: np.power(float(base), -np.arange(head_dim // 2) / head_dim)


MUTANTS = [m_levels_pow2, m_round_half_up, m_clamp_off_by_one, m_zero_is_max, m_unrounded_grid,
           m_meta_truncate, m_axis_swapped, m_pack_msb_first, m_dequant_midrise, m_softmax_no_scale,
           m_gqa_modulo, m_weights_unnormalised, m_residual_dropped, m_meta_bytes_halved,
           m_window_rounds_up, m_window_no_sinks, m_window_keys_only, m_window_exact_tokens,
           m_rope_sign, m_rope_interleaved, m_rope_freq_exponent]


@pytest.mark.parametrize("mutant", MUTANTS, ids=lambda f: f.__name__)
def test_mutant_is_caught(mutant):
    o = fresh_oracle()
    mutant(o)
    caught = []
    for check in oracle_pins.ALL_CHECKS:
        try:
            check(o)
        except Exception:  # AssertionError, or a crash caused by the planted slip
            caught.append(check.__name__)
    assert caught, f"no pin catches {mutant.__name__}"
