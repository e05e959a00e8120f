"""Seeded synthetic KV-cache workloads.

This module only draws inputs: shapes, lengths, bit widths and the raw
key/value/query tensors. It holds none of the quantization or attention
arithmetic, so both the HIP path and the CPU oracle can take their inputs from
it without sharing any of the method.

The value structure follows the pages: keys carry large magnitudes in a few
fixed channels that are the same for every token of a sequence and differ
between heads (unite.ai, "O Seu Cache KV Nao Tem um Problema de Bits...",
sections "Chaves: Os Valores Extremos Vivem em Canais Fixos" and "Embebedos
Rotatorios Complicam as Chaves"); values are flat, with no outlier channel
(section "Valores: Onde a Intuicao Quebra"). Shapes stand in for the model
families the pages discuss (GPT-2 small with 64-channel heads and a
Llama-2-7B-like cache with 2-bit KIVI-style groups of 32; a long 262,144-token
grouped-query cache with 256-channel heads from hatterialabs.com, "Asymetrie
kvantizace KV cache"). No dataset, prompt or trained weight is used.

Random streams: per-channel magnitudes, lengths and bit pairs come from numpy
PCG64 (identical on every machine); the bulk normal draws come from a
torch.Generator on the target device (deterministic per device type).
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field, replace

import numpy as np
import torch

AXIS_CHANNEL = 0
AXIS_TOKEN = 1

DTYPES = {"f32": torch.float32, "f16": torch.float16, "bf16": torch.bfloat16}

BIT_PAIRS_MIXED = ((2, 2), (3, 3), (4, 4), (6, 4), (4, 8))


@dataclass(frozen=True)
class Workload:
    name: str
    num_seqs: int
    layers: int
    kv_heads: int
    q_heads: int
    head_dim: int
    in_dtype: str  # "f32" | "f16" | "bf16"
    group_k: int
    group_v: int
    bits: tuple  # one (bits_k, bits_v) per sequence
    lengths: tuple  # cached tokens per sequence before the decode step
    new_tokens: int  # tokens appended per sequence in one decode step
    k_dist: str  # key channel-magnitude recipe, see channel_magnitudes
    v_dist: str  # "normal" | "token_lognormal"
    seed: int
    axis_k: int = AXIS_CHANNEL
    axis_v: int = AXIS_TOKEN
    notes: str = ""
    extra: dict = field(default_factory=dict, compare=False, hash=False)

    @property
    def group_size(self):  # query heads per kv head
        return self.q_heads // self.kv_heads

    @property
    def softmax_scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)

    @property
    def torch_dtype(self):
        return DTYPES[self.in_dtype]

    def scaled(self, **kw) -> "Workload":
        return replace(self, **kw)


def _uniform_bits(n, pair):
    return tuple([tuple(pair)] * n)


def tiny() -> Workload:
    """Batch 1, 1 layer, 2 kv heads, head_dim 64, 256 cached tokens, fp32; K 2-bit
    per-channel over 32-token blocks, V 2-bit per-token over 32-channel groups;
    2 of 64 key channels scaled 30x."""
    return Workload("tiny", 1, 1, 2, 2, 64, "f32", 32, 32, _uniform_bits(1, (2, 2)),
                    (256,), 1, "tiny_30x", "normal", seed=1001)


def gpt2_small() -> Workload:
    """GPT-2-small-shaped cache: 8 sequences, 12 layers, 12 heads of 64 channels,
    1024 cached tokens, fp16; K 6-bit per-channel over 64-token blocks, V 4-bit
    per-token over one 64-channel head; ~3% (2 of 64) key channels with
    lognormal(2, 0.5) magnitudes."""
    return Workload("gpt2-small", 8, 12, 12, 12, 64, "f16", 64, 64, _uniform_bits(8, (6, 4)),
                    (1024,) * 8, 1, "gpt2_lognormal", "normal", seed=1002)


def llama2_7b() -> Workload:
    """Llama-2-7B-shaped cache: 16 sequences, 32 heads of 128 channels, 4096 cached
    tokens, fp16, KIVI-style 2-bit with groups of 32 (K per-channel, V per-token),
    fp16 step/zero; channel magnitudes lognormal(0, 1) with 1% of channels 20x.
    One layer is one timed step; ``layers`` is how many independent layer
    caches a benchmark rotates through."""
    return Workload("llama2-7b", 16, 1, 32, 32, 128, "f16", 32, 32, _uniform_bits(16, (2, 2)),
                    (4096,) * 16, 1, "llama_lognormal_1pct20x", "normal", seed=1003)


def long_gqa() -> Workload:
    """One 262,144-token sequence, 32 query heads over 2 kv heads of 256 channels,
    bf16; K 4-bit, V 8-bit, groups of 32; 2% key channels at 10-50x; values with
    a lognormal per-token scale."""
    return Workload("long-gqa", 1, 1, 2, 32, 256, "bf16", 32, 32, _uniform_bits(1, (4, 8)),
                    (262144,), 1, "gqa_2pct_10_50x", "token_lognormal", seed=1004)


def mixed_batch() -> Workload:
    """64 sequences with lengths uniform in [512, 32768], 64 query heads over 8 kv
    heads of 128 channels, fp16; per-sequence (K, V) bits from
    {(2,2),(3,3),(4,4),(6,4),(4,8)}, groups of 32; 2% outlier key channels with
    lognormal magnitudes capped at 40x; 16 tokens appended per sequence."""
    rng = np.random.Generator(np.random.PCG64(1005))
    lens = tuple(int(x) for x in rng.integers(512, 32768, size=64, endpoint=True))
    bits = tuple(BIT_PAIRS_MIXED[int(i)] for i in rng.integers(0, 5, size=64))
    return Workload("mixed", 64, 1, 8, 64, 128, "f16", 32, 32, bits, lens, 16,
                    "mixed_2pct_lognormal40", "normal", seed=1005)


ALL = {"tiny": tiny, "gpt2-small": gpt2_small, "llama2-7b": llama2_7b,
       "long-gqa": long_gqa, "mixed": mixed_batch}


def get(name: str) -> Workload:
    return ALL[name]()


# ----------------------------------------------------------------------------
# Draws
# ----------------------------------------------------------------------------

def channel_magnitudes(w: Workload, layer: int) -> np.ndarray:
    """Per (kv head, channel) key magnitude, float32 [Hkv][D]; fixed channels
    per head, shared by every sequence and token of the layer."""
    rng = np.random.Generator(np.random.PCG64([w.seed, 17, layer]))
    H, D = w.kv_heads, w.head_dim
    m = np.ones((H, D), dtype=np.float64)
    for h in range(H):
        if w.k_dist == "tiny_30x":
            m[h, rng.choice(D, 2, replace=False)] = 30.0
        elif w.k_dist == "gpt2_lognormal":
            n = max(1, round(0.03 * D))
            m[h, rng.choice(D, n, replace=False)] = rng.lognormal(2.0, 0.5, n)
        elif w.k_dist == "llama_lognormal_1pct20x":
            m[h] = rng.lognormal(0.0, 1.0, D)
            n = max(1, round(0.01 * D))
            m[h, rng.choice(D, n, replace=False)] *= 20.0
        elif w.k_dist == "gqa_2pct_10_50x":
            n = max(1, round(0.02 * D))
            m[h, rng.choice(D, n, replace=False)] = rng.uniform(10.0, 50.0, n)
        elif w.k_dist == "mixed_2pct_lognormal40":
            n = max(1, round(0.02 * D))
            m[h, rng.choice(D, n, replace=False)] = np.clip(rng.lognormal(math.log(8.0), 0.75, n), 1.0, 40.0)
        elif w.k_dist == "unit":
            pass
        else:
            raise ValueError(w.k_dist)
    return m.astype(np.float32)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(int(seed) & 0x7FFFFFFFFFFFFFFF)
    return g


def draw_kv(w: Workload, layer: int, counts, *, device="cpu", stream: int = 0, dtype=None):
    """Draw ``sum(counts)`` new key and value rows for one layer, packed
    sequence-major as [sum counts][Hkv][D] in the input dtype (the layout the
    append call takes). ``stream`` separates independent draws (0 = the cached
    prefix, 1.. = appended tokens of later decode steps)."""
    n = int(sum(counts))
    H, D = w.kv_heads, w.head_dim
    dt = dtype or w.torch_dtype
    g = _gen(device, w.seed * 1_000_003 + layer * 7919 + stream * 104729)
    k = torch.randn((n, H, D), generator=g, device=device, dtype=torch.float32)
    m = torch.from_numpy(channel_magnitudes(w, layer)).to(device)
    k.mul_(m)
    v = torch.randn((n, H, D), generator=g, device=device, dtype=torch.float32)
    if w.v_dist == "token_lognormal":
        u = torch.randn((n, H, 1), generator=g, device=device, dtype=torch.float32).exp_()
        v.mul_(u)
    elif w.v_dist != "normal":
        raise ValueError(w.v_dist)
    return k.to(dt), v.to(dt)


def draw_q(w: Workload, layer: int, *, device="cpu", step: int = 0, dtype=None):
    """Decode queries [S][Hq][D] (N(0,1), input dtype)."""
    g = _gen(device, w.seed * 7_000_003 + layer * 31 + step * 977 + 5)
    q = torch.randn((w.num_seqs, w.q_heads, w.head_dim), generator=g, device=device, dtype=torch.float32)
    return q.to(dtype or w.torch_dtype)


def seq_offsets(counts):
    """Start row of each sequence inside a packed [sum counts] tensor."""
    off = [0]
    for c in counts:
        off.append(off[-1] + int(c))
    return off
