"""The error-budget workload (error_budget.py): its metric helpers on inputs
with known answers (CPU), and its GPU-measured metrics against the same
metrics computed from the oracle's reconstruction of the same inputs (GPU)."""

import math

import numpy as np
import pytest

import error_budget as eb


def test_rel_err_known_values():
    x = np.arange(1.0, 7.0).reshape(2, 3)
    assert eb.rel_err(x, x) == 0.0
    assert eb.rel_err(2 * x, x) == pytest.approx(1.0)
    assert eb.rel_err(x + 1e-3 * np.sign(x), x) == pytest.approx(1e-3 * math.sqrt(6) / np.linalg.norm(x))


def test_attention_closed_forms():
    rng = np.random.default_rng(0)
    v = rng.normal(size=(2, 9, 4))
    q = rng.normal(size=(2, 4))
    k_same = np.broadcast_to(rng.normal(size=(2, 1, 4)), (2, 9, 4))
    out, logits, w = eb.softmax_attention(q, k_same, v, 0.5)
    np.testing.assert_allclose(w, 1.0 / 9)  # equal keys: uniform weights, the mean of the values
    np.testing.assert_allclose(out, v.mean(axis=1), rtol=1e-12)
    # one key far ahead of the others takes all the weight
    k = np.zeros((2, 9, 4))
    k[:, 4] = 100.0 * q
    out, _, w = eb.softmax_attention(q, k, v, 1.0)
    np.testing.assert_allclose(out, v[:, 4], rtol=1e-9)
    assert eb.top_mass(w, 0.05) == pytest.approx(1.0)
    assert eb.top_mass(np.full((1, 100), 0.01), 0.05) == pytest.approx(0.05)


@pytest.mark.gpu
@pytest.mark.parametrize("axes,window,sinks", [((eb.CH, eb.TOK), 0, 0), ((eb.TOK, eb.CH), 0, 0),
                                               ((eb.CH, eb.TOK), 64, 32)])
def test_gpu_metrics_match_the_oracle(axes, window, sinks):
    import torch

    from bit_kv_cache_groupwise_amd import workloads as W
    from tests import gpu_helpers as H

    ak, av = axes
    w = W.llama2_7b().scaled(name="error-budget", num_seqs=2, kv_heads=2, q_heads=2, lengths=(256, 256),
                             bits=((2, 2),) * 2, axis_k=ak, axis_v=av, v_dist="token_lognormal")
    r = eb.run_config(w, window=window, sinks=sinks)
    k, v = W.draw_kv(w, 0, w.lengths, device="cuda", stream=0)
    q = W.draw_q(w, 0, device="cuda").double().cpu().numpy()
    k = k.float().cpu().numpy()
    v = v.float().cpu().numpy()
    T = w.lengths[0]
    kn2 = kd2 = vn2 = vd2 = 0.0
    outs = []
    for s in range(w.num_seqs):
        ks, vs = k[s * T:(s + 1) * T], v[s * T:(s + 1) * T]
        encs = [H.encode_window(w, ks, vs, s, h, window, sinks) if window or sinks else H.encode(w, ks, vs, s, h)
                for h in range(w.kv_heads)]
        kh = np.stack([e["k_hat"] for e in encs])
        vh = np.stack([e["v_hat"] for e in encs])
        kx = ks.astype(np.float64).transpose(1, 0, 2)
        vx = vs.astype(np.float64).transpose(1, 0, 2)
        kn2 += np.sum(kx ** 2)
        kd2 += np.sum((kh - kx) ** 2)
        vn2 += np.sum(vx ** 2)
        vd2 += np.sum((vh - vx) ** 2)
        o_ref, _, _ = eb.softmax_attention(q[s], kx, vx, w.softmax_scale)
        o_deq, _, _ = eb.softmax_attention(q[s], kh, vh, w.softmax_scale)
        outs.append(np.mean(np.linalg.norm(o_deq - o_ref, axis=1) / np.linalg.norm(o_ref, axis=1)))
    assert r["k_recon_rel"] == pytest.approx(math.sqrt(kd2 / kn2), rel=1e-9)
    assert r["v_recon_rel"] == pytest.approx(math.sqrt(vd2 / vn2), rel=1e-9)
    assert r["out_rel_dequant"] == pytest.approx(float(np.mean(outs)), rel=1e-9)
    # the fused decode (per-channel values: the generic split kernel) sits within
    # its tolerance of the dequantized attention
    assert abs(r["out_rel_fused"] - r["out_rel_dequant"]) <= 2e-3


@pytest.mark.gpu
def test_whole_vector_groups_match_the_oracle():
    """Whole-vector granularity (one step per token over every kv head's
    channels): the reconstruction the workload measures is the oracle's token-axis
    quantization of the concatenated heads, split back into heads."""
    import torch  # noqa: F401

    from bit_kv_cache_groupwise_amd import workloads as W
    from oracle import kvq_oracle as o

    w = W.llama2_7b().scaled(name="granularity", num_seqs=2, kv_heads=2, q_heads=2, lengths=(64, 64),
                             axis_k=eb.TOK, axis_v=eb.TOK, bits=((3, 3),) * 2, v_dist="token_lognormal")
    r = eb.run_config(w, whole_vector=True)
    k, v = W.draw_kv(w, 0, w.lengths, device="cuda", stream=0)
    k = k.float().cpu().numpy()
    v = v.float().cpu().numpy()
    T, HD = 64, 2 * w.head_dim
    kn2 = kd2 = vn2 = vd2 = 0.0
    for s in range(2):
        ks, vs = k[s * T:(s + 1) * T].reshape(T, HD), v[s * T:(s + 1) * T].reshape(T, HD)
        e = o.encode_head(ks, vs, group_k=HD, group_v=HD, axis_k=o.AXIS_TOKEN, axis_v=o.AXIS_TOKEN, bits_k=3,
                          bits_v=3)
        kn2 += np.sum(ks.astype(np.float64) ** 2)
        kd2 += np.sum((e["k_hat"] - ks) ** 2)
        vn2 += np.sum(vs.astype(np.float64) ** 2)
        vd2 += np.sum((e["v_hat"] - vs) ** 2)
    assert r["k_recon_rel"] == pytest.approx(math.sqrt(kd2 / kn2), rel=1e-9)
    assert r["v_recon_rel"] == pytest.approx(math.sqrt(vd2 / vn2), rel=1e-9)
    assert r["group_k"] == "vector" and r["out_rel_fused"] is None
