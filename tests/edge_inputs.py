"""Adversarial inputs for the quantizer: groups of values placed where the
method's rounding, clamping and degenerate cases sit. Inputs only: nothing
here computes a code, a step or an expected value (the oracle does that, and
``tests/oracle_pins.py`` pins the oracle on these same groups with exact
rational arithmetic).

The cases follow the quantizer's definition ([U] "O Que o Erro de
Quantizacao E Realmente Feito": zero = group minimum, step = range / (2^B - 1),
nearest step, error at most half a step; [N] "Scale menentukan sistem
koordinat kuantisasi": out-of-range values are clamped; the step and zero are
stored in fp16):

  constant groups (stored step 0), fp16-subnormal steps whose rounding makes
  the top of the group clamp, steps that underflow to 0 in fp16, exact ties
  t = k + 1/2 against a power-of-two step, near ties (t a few float32 ulps
  from k + 1/2) against a step with no exact reciprocal, minima that fp16
  rounds above the
  group (negative t, clamped to 0), bf16 and fp32 magnitudes below fp16's
  normal range (and below its smallest subnormal), magnitudes near +-65504,
  a 7000x outlier among small values, and plain normal draws.

Every group is exactly representable in the input dtype it is made for
(``representable``), so the library and the oracle see the same numbers.
"""

from __future__ import annotations

import numpy as np
import torch

G = 32  # values per group in these cases (the group size the tests use)

TORCH = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}


def to_dtype(x, dtype: str) -> np.ndarray:
    """float32 values rounded (nearest-even) to the input dtype, back as float32."""
    t = torch.from_numpy(np.ascontiguousarray(np.asarray(x, np.float32))).to(TORCH[dtype])
    return t.float().numpy()


def representable(x, dtype: str) -> bool:
    x = np.asarray(x, np.float32)
    return bool(np.array_equal(to_dtype(x, dtype).view(np.uint32), x.view(np.uint32)))


def _fill(vals, rng) -> np.ndarray:
    """32 values: the given ones (at most 32), the rest repeated from them, shuffled."""
    vals = np.asarray(vals, np.float32)
    reps = np.resize(vals, G)
    reps[:len(vals)] = vals[:G]
    return rng.permutation(reps).astype(np.float32)


def _ties(bits, dtype, z0, s0, rng):
    """z0, z0 + L*s0 (min and max), and z0 + (k + 1/2)*s0 for every k whose value
    the dtype holds exactly: t = k + 1/2 exactly when s0 is a power of two."""
    L = (1 << bits) - 1
    cand = [z0 + (k + 0.5) * s0 for k in range(L)]
    keep = [c for c in cand if representable([c], dtype)]
    if len(keep) > G - 2:
        keep = list(rng.choice(keep, G - 2, replace=False))
    return _fill([z0, z0 + L * s0, *keep], rng)


def _step_units(x: float, dtype: str, j: int) -> float:
    """The value j units in the last place of the dtype away from x (x nonzero,
    representable; the step keeps the sign of x)."""
    if dtype == "f32":
        u = np.array([x], np.float32).view(np.int32)
        return float((u + np.int32(j)).view(np.float32)[0])
    t = torch.tensor([x], dtype=TORCH[dtype]).view(torch.int16)
    return float((t + j).view(TORCH[dtype]).float()[0])


def _near_ties(bits, dtype, m, e, rng):
    """Values a few units in the dtype's last place either side of the tie
    points z0 + (k + 1/2)*s0, and ones 2^-14..2^-12 steps from them, for a
    step s0 = m * 2^e (m odd, so s0 is not a power of two and has no exact
    reciprocal) that the group stores exactly: z0 and z0 + L*s0, the minimum
    and maximum, are both held by the dtype and by fp16. Where the dtype
    allows it (fp32), the quotient t then lands within a few float32 ulps of
    k + 1/2, on both sides."""
    L = (1 << bits) - 1
    s0 = m * 2.0 ** e
    z_opts = [0.0] + [-(L * m - 2 ** p) * 2.0 ** e for p in range(24) if 2 ** p < L * m]
    z0 = next(z for z in z_opts if representable([z, z + L * s0], dtype) and representable([z], "f16"))
    top = z0 + L * s0
    cand = set()
    for k in range(L):
        p = z0 + (k + 0.5) * s0
        base = float(to_dtype([p], dtype)[0])
        pts = [base] + [float(to_dtype([p + d * s0], dtype)[0])
                        for d in (2.0 ** -14, -2.0 ** -14, 2.0 ** -13, -2.0 ** -13, 2.0 ** -12, -2.0 ** -12)]
        for b in pts:
            for j in (-2, -1, 0, 1, 2):
                v = _step_units(b, dtype, j) if b != 0.0 else b
                if z0 < v < top and (v > 0) == (b > 0):
                    cand.add(v)
    cand = sorted(cand)
    if len(cand) > G - 2:
        cand = list(rng.choice(cand, G - 2, replace=False))
    return _fill([z0, top, *cand], rng)


def groups(bits: int, dtype: str, seed: int = 0):
    """(name, float32[32]) adversarial groups for a bit width and input dtype."""
    rng = np.random.Generator(np.random.PCG64([seed, bits, {"f32": 0, "f16": 1, "bf16": 2}[dtype]]))
    L = (1 << bits) - 1
    tiny = 2.0 ** -24  # fp16's smallest subnormal
    out = [
        ("const_pos", np.full(G, 1.5, np.float32)),
        ("const_neg", np.full(G, -3.25, np.float32)),
        ("const_zero", np.zeros(G, np.float32)),
        ("const_negzero", np.full(G, -0.0, np.float32)),
        ("ties_unit", _ties(bits, dtype, -2.0, 1.0 / 8, rng)),
        ("ties_small", _ties(bits, dtype, 0.25 if dtype != "bf16" else 0.0, 2.0 ** -12, rng)),
        ("ties_neg", _ties(bits, dtype, -40.0, 0.5, rng)),
        ("neartie_m3", _near_ties(bits, dtype, 3, -8, rng)),
        ("neartie_m5", _near_ties(bits, dtype, 5, -4, rng)),
    ]
    # fp16-subnormal steps: range M * 2^-24 with M a little above L, so the
    # stored step rounds down and the top of the group clamps
    for M in sorted({L + 1, L + max(1, L // 2), 2 * L - 1}):
        if M < 256 or dtype != "bf16":
            k = np.concatenate([[0, M], rng.integers(0, M + 1, G - 2)])
            out.append((f"substep_{M}", _fill(k * tiny, rng)))
    # steps that underflow to 0 in fp16 (range below half the smallest subnormal times L)
    out.append(("underflow_zero_base", _fill([0.0, tiny] * 16, rng)))
    out.append(("underflow_base5", _fill([5 * tiny, 6 * tiny] * 16, rng)))
    # magnitudes below fp16's normal range (2^-14) and below its smallest subnormal
    for base in (3.0e-7, 2.0 ** -20, 1.0e-9):
        v = to_dtype(base * (1.0 + np.arange(G) / 64.0), dtype)
        out.append((f"tiny_{base:.0e}", _fill(v, rng)))
    # near the fp16 limit: +-65000 (as the dtype holds it), a narrow group near the top
    big = float(to_dtype([65000.0], dtype)[0])
    top = 65504.0 if dtype != "bf16" else 65280.0
    mid = to_dtype(rng.uniform(-big, big, G - 2), dtype)
    out.append(("big_pm65000", _fill([-big, big, *mid], rng)))
    out.append(("big_top", _fill(to_dtype(np.linspace(top - 2048.0, top, G), dtype), rng)))
    # an outlier 7000x above small values ([U] "Chaves: Os Valores Extremos Vivem em Canais Fixos")
    small = to_dtype(rng.normal(0.0, 0.3, G - 1), dtype)
    out.append(("outlier_7000", _fill([float(to_dtype([7000.0], dtype)[0]), *small], rng)))
    if dtype == "f32":
        # fp32 minima that fp16 rounds above the group: negative t, clamped to 0
        out.append(("zero_rounds_up", _fill(1000.3 + np.arange(G) * 0.001, rng)))
        out.append(("zero_rounds_up_small", _fill(0.1 + np.arange(G) * 1.0e-6, rng)))
        # an fp32 range far below fp16's smallest step around 1e-3
        out.append(("underflow_f32", _fill(1.0e-3 + np.arange(G) * 2.0 ** -33, rng)))
    out.append(("normal", to_dtype(rng.normal(0.0, 1.0, G), dtype)))
    for name, g in out:
        assert g.shape == (G,) and representable(g, dtype), (name, dtype)
        assert np.all(np.abs(g) <= 65504.0), name
    return out


def tensor(bits: int, dtype: str, axis: int, tokens: int, head_dim: int, seed: int,
           max_abs: float = 65504.0) -> np.ndarray:
    """float32 [tokens][head_dim]: every group of the given axis (0: a channel
    over a G-token block; 1: G consecutive channels of a token) takes one of the
    adversarial groups in turn (those whose values stay within max_abs); tokens
    past the last whole block (channel axis) are normal draws with a few extreme
    values (they stay in the residual)."""
    gs = [g for g in groups(bits, dtype, seed) if np.abs(g[1]).max() <= max_abs]
    rng = np.random.Generator(np.random.PCG64([seed, 99, bits]))
    x = to_dtype(rng.normal(0.0, 1.0, (tokens, head_dim)), dtype)
    order = rng.permutation(len(gs))
    i = 0
    if axis == 0:
        for b in range(tokens // G):
            for c in range(head_dim):
                x[b * G:(b + 1) * G, c] = gs[order[i % len(gs)]][1]
                i += 1
        tail = tokens - (tokens // G) * G
        if tail:
            x[tokens - tail, 0] = float(to_dtype([-min(65000.0, max_abs)], dtype)[0])
            x[tokens - 1, head_dim - 1] = float(to_dtype([3.0e-7], dtype)[0])
    else:
        for t in range(tokens):
            for g in range(head_dim // G):
                x[t, g * G:(g + 1) * G] = gs[order[i % len(gs)]][1]
                i += 1
    return x
