"""CPU oracle: groupwise asymmetric integer quantization of a transformer KV
cache, the bit-packed storage of its codes, fp64 dequantization, and the
decode-step softmax attention that reads the cache.

TEST INFRASTRUCTURE. Only ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` may import this module. The product path
(the HIP library and its Python binding) never imports, calls or links it, and
this module imports nothing from the product. It is deliberately plain and
slow: numpy elementwise float32 operations in the order the method states them,
float64 for everything after the codes, and library primitives (matmul,
exp, min/max) only as single steps.

Sources, cited by page title and section heading:

  [N] nalar.dev, "Kuantisasi KV cache untuk mengurangi memory inferensi
      long-context"
  [U] unite.ai (Portuguese edition), "O Seu Cache KV Nao Tem um Problema de
      Bits. Tem um Problema de Geometria."
  [H] hatterialabs.com (Czech), "Asymetrie kvantizace KV cache"

What the pages fix, restated:
  * a group's zero point is its minimum and its step is its range divided by
    2^B - 1; every element is rounded to the nearest step, so the error of an
    element is at most half a step ([U] "O Que o Erro de Quantizacao E
    Realmente Feito");
  * values outside the representable range are clamped ([N] "Scale menentukan
    sistem koordinat kuantisasi");
  * keys take one step per channel (the group runs along tokens), values one
    step per token (the group runs along channels) ([U] "Chaves: Os Valores
    Extremos Vivem em Canais Fixos", "Valores: Onde a Intuicao Quebra");
  * a per-channel step needs tokens that have not arrived yet, so recent key
    tokens stay unquantized until a whole group has accumulated ([U] "O Imposto
    dos Sistemas e Por Que Nao E um Detalhe"; [N] "Pengecualian recent-token
    mengubah perhitungan memory");
  * cache elements = 2 * layers * cached_tokens * kv_heads * head_dim ([N]
    "Ukuran cache bertambah mengikuti token, layer, dan KV head");
  * decode attention reads every cached key and value once per generated token
    ([U] "Por Que o Cache KV E Onde Isso Morde").

Readings taken where the pages are silent (each one is also listed with its
reason in the design notes of the repository):
  R1 the nearest step is found with round-half-to-even on t = (x - z) / s;
  R2 step and minimum are computed in float32 (a float32 subtract and a
     correctly rounded float32 divide, no fused multiply-add), then each is
     rounded once, to nearest-even, to the metadata type (fp16 by default);
     codes are computed against the stored (rounded) step and zero, so the
     quantizer and the dequantizer use one grid;
  R3 a group whose stored step is 0 (max == min, or a step below fp16's
     smallest subnormal) gets code 0 everywhere and reconstructs to its zero;
  R4 with the channel axis, tokens [floor(len/G)*G, len) stay in the input
     dtype (the residual); nothing else is kept unquantized;
  R5 codes are packed as a dense little-endian bitstream per unit of 32
     channels (see pack_rows); the pages name the packing layout as a free
     format parameter ([N] "Scale menentukan sistem koordinat kuantisasi");
  R6 one decode step first appends the new token, then attends to every
     cached token including it; query head h reads kv head h // (Hq/Hkv).
"""

from __future__ import annotations

import numpy as np

AXIS_CHANNEL = 0  # one (step, zero) per channel per block of G consecutive tokens
AXIS_TOKEN = 1  # one (step, zero) per token per group of G consecutive channels
SUPPORTED_BITS = (2, 3, 4, 6, 8)


def levels(bits: int) -> int:
    """Largest code, 2^B - 1 ([U] "O Que o Erro de Quantizacao ...")."""
    return (1 << bits) - 1


def to_meta(v, meta_dtype: str = "f16") -> np.ndarray:
    """Round float32 values to the metadata type, returned as float32 (R2).

    numpy's float32 -> float16 cast rounds to nearest, ties to even."""
    v = np.asarray(v, dtype=np.float32)
    if meta_dtype == "f16":
        return v.astype(np.float16).astype(np.float32)
    if meta_dtype == "f32":
        return v
    raise ValueError(f"unknown metadata dtype {meta_dtype!r}")


def group_params(mn, mx, bits: int, meta_dtype: str = "f16"):
    """Stored (step, zero) of groups with float32 minimum ``mn`` and maximum ``mx``.

    zero = group minimum; step = (max - min) / (2^B - 1), computed as a float32
    subtraction followed by a float32 division ([U] "O Que o Erro de
    Quantizacao ..."), then both rounded to the metadata type (R2)."""
    mn = np.asarray(mn, dtype=np.float32)
    mx = np.asarray(mx, dtype=np.float32)
    rng = mx - mn  # float32
    step32 = rng / np.float32(levels(bits))  # float32, correctly rounded
    return to_meta(step32, meta_dtype), to_meta(mn, meta_dtype)


def encode_values(x, s, z, bits: int) -> np.ndarray:
    """Codes of float32 values ``x`` on the grid z + k*s, k in [0, 2^B - 1].

    t = (x - z) / s in float32; code = clamp(round_half_even(t), 0, 2^B - 1)
    ([U] "O Que o Erro ...": nearest step; [N] "Scale menentukan ...": clamp);
    code 0 where the stored step is 0 (R3). ``s`` and ``z`` broadcast to x."""
    x = np.asarray(x, dtype=np.float32)
    s = np.asarray(s, dtype=np.float32)
    z = np.asarray(z, dtype=np.float32)
    s_div = np.where(s == 0, np.float32(1), s).astype(np.float32)
    t = (x - z) / s_div  # float32 subtract, float32 divide
    k = np.clip(np.rint(t), 0, levels(bits))  # rint: round half to even (R1)
    k = np.where(s == 0, 0, k)
    return k.astype(np.uint8)


def quantize_tensor(x, axis: int, group: int, bits: int, meta_dtype: str = "f16"):
    """Quantize the cached rows of one tensor of one (layer, sequence, kv head).

    ``x``: float32 [T][D], token-major. Returns (codes uint8 [Tq][D],
    step float32, zero float32, residual float32 [T - Tq][D]).

    AXIS_CHANNEL (keys, [U] "Chaves ..."): block b holds tokens [bG, bG+G);
    each (block, channel) is one group of G values; step/zero are
    [Tq/G][D]; Tq = floor(T/G)*G and the tail stays unquantized (R4,
    [U] "O Imposto dos Sistemas ...").
    AXIS_TOKEN (values, [U] "Valores ..."): each (token, channel group g)
    holds channels [gG, gG+G); step/zero are [T][D/G]; Tq = T."""
    x = np.asarray(x, dtype=np.float32)
    T, D = x.shape
    if axis == AXIS_CHANNEL:
        nb = T // group
        tq = nb * group
        xb = x[:tq].reshape(nb, group, D)  # [block][token in block][channel]
        mn = xb.min(axis=1)
        mx = xb.max(axis=1)
        s, z = group_params(mn, mx, bits, meta_dtype)
        codes = encode_values(xb, s[:, None, :], z[:, None, :], bits).reshape(tq, D)
        return codes, s, z, x[tq:].copy()
    if axis == AXIS_TOKEN:
        if D % group:
            raise ValueError("token-axis group must divide head_dim")
        xg = x.reshape(T, D // group, group)  # [token][group][channel in group]
        mn = xg.min(axis=2)
        mx = xg.max(axis=2)
        s, z = group_params(mn, mx, bits, meta_dtype)
        codes = encode_values(xg, s[..., None], z[..., None], bits).reshape(T, D)
        return codes, s, z, x[T:].copy()
    raise ValueError(f"unknown axis {axis}")


def dequantize_tensor(codes, s, z, resid, axis: int, group: int) -> np.ndarray:
    """float64 reconstruction x_hat = z + code * s of every cached row, followed by
    the residual rows as they were stored ([N] "Scale menentukan ...": x_hat is
    the approximation used by the computation that follows).

    With fp16 metadata z + code*s is exact in float64, so float32(x_hat) is the
    correctly rounded value of the exact reconstruction."""
    codes = np.asarray(codes, dtype=np.float64)
    tq, D = codes.shape
    s = np.asarray(s, dtype=np.float64)
    z = np.asarray(z, dtype=np.float64)
    if axis == AXIS_CHANNEL:
        nb = tq // group
        xq = z[:, None, :] + codes.reshape(nb, group, D) * s[:, None, :]
        xq = xq.reshape(tq, D)
    else:
        xq = z[..., None] + codes.reshape(tq, D // group, group) * s[..., None]
        xq = xq.reshape(tq, D)
    return np.concatenate([xq, np.asarray(resid, dtype=np.float64)], axis=0)


# ----------------------------------------------------------------------------
# Storage format (R5). The pages leave the packing layout open ([N] "Scale
# menentukan sistem koordinat kuantisasi" lists it among the format parameters).
# ----------------------------------------------------------------------------

def pack_rows(codes, bits: int) -> np.ndarray:
    """Pack uint8 codes [N][D] (D % 32 == 0) into uint32 words [N][D*B/32].

    A row is D/32 units; unit u is B consecutive words holding channels
    32u..32u+31. Channel 32u+j occupies bits [j*B, (j+1)*B) of the unit's
    32*B-bit stream, whose bit i is bit (i mod 32) of the unit's word i // 32.
    3- and 6-bit codes straddle words; there is no padding."""
    codes = np.asarray(codes)
    N, D = codes.shape
    if D % 32:
        raise ValueError("head_dim must be a multiple of 32")
    units = codes.reshape(N, D // 32, 32).astype(np.uint64)
    words = np.zeros((N, D // 32, bits), dtype=np.uint64)
    mask32 = np.uint64(0xFFFFFFFF)
    for j in range(32):
        w, sh = divmod(j * bits, 32)
        words[:, :, w] |= (units[:, :, j] << np.uint64(sh)) & mask32
        if sh + bits > 32:
            words[:, :, w + 1] |= units[:, :, j] >> np.uint64(32 - sh)
    return words.reshape(N, (D // 32) * bits).astype(np.uint32)


def unpack_rows(words, bits: int, D: int) -> np.ndarray:
    """Inverse of pack_rows."""
    words = np.asarray(words, dtype=np.uint64)
    N = words.shape[0]
    wu = words.reshape(N, D // 32, bits)
    out = np.zeros((N, D // 32, 32), dtype=np.uint64)
    mask = np.uint64(levels(bits))
    for j in range(32):
        w, sh = divmod(j * bits, 32)
        v = wu[:, :, w] >> np.uint64(sh)
        if sh + bits > 32:
            v |= wu[:, :, w + 1] << np.uint64(32 - sh)
        out[:, :, j] = v & mask
    return out.reshape(N, D).astype(np.uint8)


def meta_words(s, z) -> np.ndarray:
    """fp16 (step, zero) pairs as uint32 words: step in the low half (lower
    address), zero in the high half."""
    sb = np.asarray(s, dtype=np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
    zb = np.asarray(z, dtype=np.float32).astype(np.float16).view(np.uint16).astype(np.uint32)
    return (sb | (zb << np.uint32(16))).astype(np.uint32)


# ----------------------------------------------------------------------------
# Attention
# ----------------------------------------------------------------------------

def attend(q, khat, vhat, scale: float) -> np.ndarray:
    """Softmax attention of R query vectors over T cached tokens, in float64.

    logits = scale * q . k_t; weights = softmax over t (max subtracted first);
    out = sum_t w_t v_t. Keys enter before the softmax, values after it
    ([N] "Key dan value dapat memiliki struktur numerik berbeda").
    With T == 0 the output is defined as 0."""
    q = np.asarray(q, dtype=np.float64)
    khat = np.asarray(khat, dtype=np.float64)
    vhat = np.asarray(vhat, dtype=np.float64)
    R, D = q.shape
    if khat.shape[0] == 0:
        return np.zeros((R, D))
    logits = float(scale) * (q @ khat.T)  # [R][T]
    logits = logits - logits.max(axis=1, keepdims=True)
    w = np.exp(logits)
    w = w / w.sum(axis=1, keepdims=True)
    return w @ vhat


def attend_heads(q, khat, vhat, scale: float) -> np.ndarray:
    """One sequence: q [Hq][D], khat/vhat [Hkv][T][D] -> out [Hq][D]; query head
    h reads kv head h // (Hq/Hkv) (R6; grouped-query attention shares kv heads
    among query heads, [N] "Ukuran cache bertambah ...")."""
    q = np.asarray(q, dtype=np.float64)
    hq = q.shape[0]
    hkv = len(khat)
    if hq % hkv:
        raise ValueError("q_heads must be a multiple of kv_heads")
    r = hq // hkv
    out = np.zeros(q.shape)
    for kv in range(hkv):
        out[kv * r:(kv + 1) * r] = attend(q[kv * r:(kv + 1) * r], khat[kv], vhat[kv], scale)
    return out


# ----------------------------------------------------------------------------
# One cached (layer, sequence, kv head): encode + dequantize, as a record
# ----------------------------------------------------------------------------

def encode_head(k, v, *, group_k: int, group_v: int, axis_k: int, axis_v: int,
                bits_k: int, bits_v: int, meta_dtype: str = "f16") -> dict:
    """Encode the full token history of one (layer, sequence, kv head).

    The result depends only on the history (R4): appending the same tokens in
    any chunking yields the same bytes. Returns packed words, metadata words,
    residual rows and the float64 reconstructions."""
    k = np.asarray(k, dtype=np.float32)
    v = np.asarray(v, dtype=np.float32)
    D = k.shape[1]
    out = {}
    for name, x, axis, group, bits in (("k", k, axis_k, group_k, bits_k),
                                       ("v", v, axis_v, group_v, bits_v)):
        codes, s, z, resid = quantize_tensor(x, axis, group, bits, meta_dtype)
        out[name + "_codes"] = codes
        out[name + "_words"] = pack_rows(codes, bits) if len(codes) else np.zeros((0, D * bits // 32), np.uint32)
        out[name + "_scale"] = s
        out[name + "_zero"] = z
        out[name + "_meta"] = meta_words(s, z) if meta_dtype == "f16" else None
        out[name + "_resid"] = resid
        out[name + "_hat"] = dequantize_tensor(codes, s, z, resid, axis, group)
    return out


# ----------------------------------------------------------------------------
# Sizes ([N] "Ukuran cache bertambah ..." and "Pengecualian recent-token ...")
# ----------------------------------------------------------------------------

def cache_elements(layers: int, cached_tokens: int, kv_heads: int, head_dim: int) -> int:
    """2 * layers * cached_tokens * kv_heads * head_dim; the 2 counts K and V."""
    return 2 * layers * cached_tokens * kv_heads * head_dim


def head_bytes(tokens: int, head_dim: int, *, group_k: int, group_v: int, axis_k: int,
               axis_v: int, bits_k: int, bits_v: int, in_bytes: int, meta_bytes: int = 4) -> dict:
    """Bytes one (layer, sequence, kv head) stores after ``tokens`` tokens, by term:
    packed codes, scale/zero metadata and the high-precision residual rows
    ([N] "Pengecualian recent-token ..." splits total memory the same way;
    workspace is not per head). ``meta_bytes`` is the size of one (step, zero) pair."""
    res = {"codes": 0, "meta": 0, "residual": 0}
    for axis, group, bits in ((axis_k, group_k, bits_k), (axis_v, group_v, bits_v)):
        if axis == AXIS_CHANNEL:
            tq = (tokens // group) * group
            res["codes"] += tq * head_dim * bits // 8
            res["meta"] += (tq // group) * head_dim * meta_bytes
            res["residual"] += (tokens - tq) * head_dim * in_bytes
        else:
            res["codes"] += tokens * head_dim * bits // 8
            res["meta"] += tokens * (head_dim // group) * meta_bytes
    res["total"] = res["codes"] + res["meta"] + res["residual"]
    return res


def effective_bits(bits_k: int, bits_v: int, group_elems_k: int, group_elems_v: int,
                   meta_bits: int = 32) -> float:
    """Average stored bits per K/V element including one (step, zero) pair per group."""
    return ((bits_k + meta_bits / group_elems_k) + (bits_v + meta_bits / group_elems_v)) / 2.0


# ----------------------------------------------------------------------------
# Full-precision recent window and attention sinks ([U] "O Imposto dos
# Sistemas e Por Que Nao E um Detalhe": the most recent tokens, up to a window
# of about 128, stay in full precision and are quantized in groups once enough
# have accumulated; [U] "O Que Fazer Com Isso": keep a full-precision window of
# recently generated tokens; [U] "Onde o Trabalho Esta Indo": InnerQ keeps
# high-precision windows for recent tokens and for attention-sink tokens; [N] "Pengecualian
# recent-token mengubah perhitungan memory": the recent part is a
# high-precision region next to the packed cache).
#
# Reading W1 (the pages give the policy, not its boundary): with a window of R
# tokens and S sink tokens, the attention reads token t in full precision when
# t < S (a sink) or t lies in the recent part; every key block of Gb tokens that
# lies wholly inside [S, len - R) is read quantized. Gb is the block length of
# the channel-axis tensor (its G; 1 when no tensor groups along tokens), and S
# is a multiple of Gb. So between R and R + Gb - 1 recent tokens are full
# precision once len >= S + R. Both tensors share the boundary. The window is
# off (R4 alone) when R == S == 0.
# ----------------------------------------------------------------------------

def token_block(axis_k: int, group_k: int, axis_v: int, group_v: int) -> int:
    """Gb: tokens per quantization block along the token axis (W1)."""
    g = [group for axis, group in ((axis_k, group_k), (axis_v, group_v)) if axis == AXIS_CHANNEL]
    return max(g) if g else 1


def full_precision_mask(length: int, window: int, sinks: int, block: int) -> np.ndarray:
    """Boolean [length]: True where the attention reads the token in full
    precision under W1. The quantized tokens are [S, Q) with
    Q = max(S, Gb * floor((len - R) / Gb))."""
    if window < 0 or sinks < 0 or sinks % block:
        raise ValueError("window >= 0, sinks >= 0 and a multiple of the block")
    t = np.arange(length)
    if window == 0 and sinks == 0:
        return np.zeros(length, dtype=bool)
    q = max(sinks, block * ((length - window) // block))  # floor division
    return (t < sinks) | (t >= q)


def apply_window(x, x_hat, mask) -> np.ndarray:
    """Rows of the float64 reconstruction where the mask is set are replaced by
    the exact input rows (W1)."""
    out = np.array(x_hat, dtype=np.float64, copy=True)
    m = np.asarray(mask, dtype=bool)
    out[m] = np.asarray(x, dtype=np.float32)[m].astype(np.float64)
    return out


def encode_head_window(k, v, *, window: int, sinks: int, group_k: int, group_v: int, axis_k: int,
                       axis_v: int, bits_k: int, bits_v: int, meta_dtype: str = "f16") -> dict:
    """encode_head plus the full-precision window: the stored codes, metadata and
    residual are unchanged (every token is still quantized as it arrives); the
    reconstructions the attention reads, ``k_hat`` and ``v_hat``, take the
    exact input rows where ``full_precision_mask`` is set. ``k_hat_q`` and
    ``v_hat_q`` keep the reconstructions without the window."""
    enc = encode_head(k, v, group_k=group_k, group_v=group_v, axis_k=axis_k, axis_v=axis_v,
                      bits_k=bits_k, bits_v=bits_v, meta_dtype=meta_dtype)
    block = token_block(axis_k, group_k, axis_v, group_v)
    mask = full_precision_mask(np.asarray(k).shape[0], window, sinks, block)
    enc["k_hat_q"], enc["v_hat_q"] = enc["k_hat"], enc["v_hat"]
    enc["k_hat"] = apply_window(k, enc["k_hat_q"], mask)
    enc["v_hat"] = apply_window(v, enc["v_hat_q"], mask)
    enc["fp_mask"] = mask
    return enc


# ----------------------------------------------------------------------------
# Pre-rotation keys ([U] "Embebedos Rotatorios Complicam as Chaves": rotary
# position embeddings turn pairs of channels by an angle that grows with the
# token's position, which spreads a fixed outlier channel into its partner;
# KVQuant's answer is to quantize the keys before the rotation and to rotate
# after dequantization).
#
# Reading P1 (the pages name the rotation, not its formula): the standard
# rotary embedding with frequencies theta_i = base^(-2i/D), i < D/2, rotating
# the channel pair (i, i + D/2) of a key at position t by the angle t*theta_i;
# positions are the token indices 0, 1, 2, ... of the cache. The query is given
# already rotated at its own position, so a score is q . rope(k_hat_t, t).
# ----------------------------------------------------------------------------

def rope_frequencies(head_dim: int, base: float) -> np.ndarray:
    """theta_i = base^(-2i/D) for i < D/2, float64 (reading P1)."""
    i = np.arange(head_dim // 2, dtype=np.float64)
    return np.power(float(base), -2.0 * i / head_dim)


def rope(x, positions, base: float) -> np.ndarray:
    """Rotate rows x[t] (float64 [T][D]) by positions[t]: channel pair
    (i, i + D/2) becomes (a cos - b sin, a sin + b cos) at angle
    positions[t] * theta_i (reading P1)."""
    x = np.asarray(x, dtype=np.float64)
    D = x.shape[1]
    h = D // 2
    ang = np.asarray(positions, dtype=np.float64)[:, None] * rope_frequencies(D, base)[None, :]
    c, s = np.cos(ang), np.sin(ang)
    a, b = x[:, :h], x[:, h:]
    return np.concatenate([a * c - b * s, a * s + b * c], axis=1)


def attend_rope(q, khat, vhat, scale: float, base: float) -> np.ndarray:
    """Attention over pre-rotation keys: the reconstructed key of token t is
    rotated to position t after dequantization, then scored against q."""
    khat = np.asarray(khat, dtype=np.float64)
    return attend(q, rope(khat, np.arange(khat.shape[0]), base), vhat, scale)
