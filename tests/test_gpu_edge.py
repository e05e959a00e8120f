"""The quantizer's edge cases on the GPU, through the C ABI, against the CPU
oracle: every bit width B in {2,3,4,6,8}, both grouping axes for both tensors,
fp32, fp16 and bf16 inputs. The groups (tests/edge_inputs.py) are constant,
have fp16-subnormal steps whose rounding makes the top clamp, steps that
underflow to 0, exact ties t = k + 1/2, near ties (t a few float32 ulps
from k + 1/2, step with no exact reciprocal), fp32 minima that fp16 rounds above the
group, magnitudes below fp16's normal range and near 65504, and a 7000x
outlier ([U] "O Que o Erro de Quantizacao E Realmente Feito": nearest step,
half-step bound; [N] "Scale menentukan sistem koordinat kuantisasi": clamp).

Packed codes, metadata, residual rows and kvq_dequantize output are compared
bit for bit; the decode attention over these caches (values on the token axis)
is compared with the fp64 oracle at the 2e-3 row tolerance. Pools, workspace
and outputs start poisoned (0xFF bytes), so an unwritten or stray byte shows."""

import sys

import numpy as np
import pytest
import torch

from bit_kv_cache_groupwise_amd import workloads as W
from oracle import kvq_oracle as o
from tests import edge_inputs as E
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu

BITS = (2, 3, 4, 6, 8)
T = 2 * E.G + 5  # two whole key blocks and 5 residual rows
SPLIT = 50  # appended as 50 rows, then 19 (the second append completes block 1 from the residual)


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _workload(dtype, axis_k, axis_v, kv_heads, q_heads, head_dim):
    return W.tiny().scaled(num_seqs=len(BITS), kv_heads=kv_heads, q_heads=q_heads, head_dim=head_dim,
                           in_dtype=dtype, group_k=E.G, group_v=E.G, axis_k=axis_k, axis_v=axis_v,
                           bits=tuple((b, b) for b in BITS), lengths=(T,) * len(BITS), new_tokens=0)


def _tensors(w, key_max_abs=65504.0):
    """float32 [S][T][Hkv][D] keys and values: adversarial groups along each
    tensor's own axis, a different arrangement per sequence and head."""
    S, Hk, D = w.num_seqs, w.kv_heads, w.head_dim
    k = np.zeros((S, T, Hk, D), np.float32)
    v = np.zeros_like(k)
    for s, (bk, bv) in enumerate(w.bits):
        for h in range(Hk):
            k[s, :, h] = E.tensor(bk, w.in_dtype, w.axis_k, T, D, seed=100 * s + 2 * h, max_abs=key_max_abs)
            v[s, :, h] = E.tensor(bv, w.in_dtype, w.axis_v, T, D, seed=100 * s + 2 * h + 1)
    return k, v


def _fill(w, k, v):
    cache = H.make_cache(w)
    dt = E.TORCH[w.in_dtype]
    for lo, hi in ((0, SPLIT), (SPLIT, T)):
        kp = torch.from_numpy(np.ascontiguousarray(k[:, lo:hi].reshape(-1, w.kv_heads, w.head_dim))).to(dt)
        vp = torch.from_numpy(np.ascontiguousarray(v[:, lo:hi].reshape(-1, w.kv_heads, w.head_dim))).to(dt)
        cache.append(0, kp.cuda(), vp.cuda(), [hi - lo] * w.num_seqs)
    torch.cuda.synchronize()
    assert cache.lengths(0) == [T] * w.num_seqs
    return cache


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("axes", [(o.AXIS_CHANNEL, o.AXIS_TOKEN), (o.AXIS_TOKEN, o.AXIS_CHANNEL)],
                         ids=["k_channel_v_token", "k_token_v_channel"])
def test_edge_groups_bit_exact(dtype, axes):
    w = _workload(dtype, axes[0], axes[1], kv_heads=2, q_heads=2, head_dim=64)
    _note(f"[edge] dtype={dtype} axes={axes} bits={BITS} T={T}")
    k, v = _tensors(w)
    cache = _fill(w, k, v)
    for s in range(w.num_seqs):
        kd, vd = cache.dequantize(0, s)
        torch.cuda.synchronize()
        kd, vd = kd.cpu().numpy(), vd.cpu().numpy()
        for h in range(w.kv_heads):
            enc = H.assert_head_bytes(cache, w, 0, s, h, k[s], v[s])
            np.testing.assert_array_equal(kd[h].view(np.uint32), enc["k_hat"].astype(np.float32).view(np.uint32),
                                          err_msg=f"dequantized keys s{s} B{w.bits[s]}")
            np.testing.assert_array_equal(vd[h].view(np.uint32), enc["v_hat"].astype(np.float32).view(np.uint32),
                                          err_msg=f"dequantized values s{s} B{w.bits[s]}")
    cache.close()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
@pytest.mark.parametrize("q_heads", [2, 8], ids=["one_query_per_head", "query_groups_of_4"])
def test_edge_groups_decode(dtype, q_heads):
    """Decode attention over caches of adversarial groups (constant and
    degenerate groups, clamped codes, values near 65504 and below 2^-14).

    Keys stay below 2^14 in magnitude (the 7000x outlier included): keys near
    65504 give logits of ~10^4, where float32 evaluation of the scores alone
    (24-bit sums, 22-bit fp16 hi + lo weights on the matrix cores) moves the
    softmax weights by ~1e-3, which is the tolerance itself. The bit-exact test
    above covers those key groups, and the values here take every group."""
    w = _workload(dtype, o.AXIS_CHANNEL, o.AXIS_TOKEN, kv_heads=2, q_heads=q_heads, head_dim=128)
    _note(f"[edge decode] dtype={dtype} q_heads={q_heads}")
    k, v = _tensors(w, key_max_abs=2.0 ** 14)
    cache = _fill(w, k, v)
    q = W.draw_q(w, 0)
    out = cache.decode(0, q.cuda(), w.softmax_scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    assert np.isfinite(out).all()
    worst = 0.0
    for s in range(w.num_seqs):
        encs = [H.assert_head_bytes(cache, w, 0, s, h, k[s], v[s]) for h in range(w.kv_heads)]
        err = H.row_rel_err(out[s], H.attn_ref(w, q[s].float().numpy(), encs))
        worst = max(worst, float(err.max()))
        assert np.all(err <= H.ATTN_TOL), (dtype, q_heads, s, w.bits[s], float(err.max()))
    _note(f"[edge decode] dtype={dtype} q_heads={q_heads} worst row rel err {worst:.3e}")
    cache.close()


@pytest.mark.parametrize("dtype", ["f32", "f16", "bf16"])
def test_tiny_value_steps_next_to_large(dtype):
    """Query groups whose rows weight tokens of very different value scales.

    Per bit width B, two sequences of one kv head and four query heads (the
    query-group kernel). In the first, query row 0 puts all of its weight on
    token 37, whose values are tiny (1e-6, 1e-5, 1e-4 times U(1, 3) at B = 2, 4,
    8: nonzero value steps below fp16's normal range), inside a 32-token tile of
    tokens with values up to 6e4 (steps ~4e4 at B = 2); rows 1-3 are orthogonal
    to row 0 and spread their weight over every token. In the second, every
    value is that small. Each row's output must meet the 2e-3 bar relative to
    its own magnitude (~1e-6 for row 0, ~1e4 for rows 1-3), which a single
    power-of-two scale shared by the rows of a tile cannot give."""
    bits = (2, 4, 8)
    w = W.tiny().scaled(num_seqs=2 * len(bits), kv_heads=1, q_heads=4, head_dim=128, in_dtype=dtype,
                        group_k=E.G, group_v=E.G, axis_k=o.AXIS_CHANNEL, axis_v=o.AXIS_TOKEN,
                        bits=tuple((b, b) for b in bits for _ in range(2)), lengths=(T,) * (2 * len(bits)),
                        new_tokens=0)
    _note(f"[edge tiny steps] dtype={dtype} bits={bits}")
    rng = np.random.Generator(np.random.PCG64(77))
    S, D, hot = w.num_seqs, w.head_dim, 37
    tiny = {2: 1.0e-6, 4: 1.0e-5, 8: 1.0e-4}
    q = rng.normal(0.0, 1.0, (S, 4, D))
    for s in range(S):  # rows 1-3 orthogonal to row 0
        q0 = q[s, 0] / np.linalg.norm(q[s, 0])
        for r in range(1, 4):
            q[s, r] -= (q[s, r] @ q0) * q0
    q = E.to_dtype(q, dtype)
    k = np.zeros((S, T, 1, D), np.float32)
    v = np.zeros((S, T, 1, D), np.float32)
    for s in range(S):
        if s % 2 == 0:
            # row 0's logit at the hot token is ~60 above every other one
            c = 60.0 / (float(q[s, 0].astype(np.float64) @ q[s, 0]) * w.softmax_scale)
            k[s, hot, 0] = E.to_dtype(c * q[s, 0], dtype)
            v[s, :, 0] = E.to_dtype(rng.uniform(-6.0e4, 6.0e4, (T, D)), dtype)
            v[s, hot, 0] = E.to_dtype(tiny[w.bits[s][1]] * rng.uniform(1.0, 3.0, D), dtype)
        else:
            k[s, :, 0] = E.to_dtype(rng.normal(0.0, 1.0, (T, D)), dtype)
            v[s, :, 0] = E.to_dtype(tiny[w.bits[s][1]] * rng.uniform(-2.0, 2.0, (T, D)), dtype)
    cache = _fill(w, k, v)
    qt = torch.from_numpy(np.ascontiguousarray(q)).to(E.TORCH[dtype])
    out = cache.decode(0, qt.cuda(), w.softmax_scale)
    torch.cuda.synchronize()
    out = out.cpu().numpy()
    for s in range(S):
        enc = H.assert_head_bytes(cache, w, 0, s, 0, k[s], v[s])
        ref = H.attn_ref(w, qt[s].float().numpy(), [enc])
        err = H.row_rel_err(out[s], ref)
        _note(f"[edge tiny steps] s{s} B{w.bits[s]} |ref| {np.abs(ref).max(axis=-1)} row err {err}")
        assert np.all(err <= H.ATTN_TOL), (dtype, s, w.bits[s], err)
    cache.close()
