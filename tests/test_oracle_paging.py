"""The oracle facts the paged cache rests on ([N] "State quantized cache harus
tetap selaras dengan posisi": moving cached tokens between physical slots --
pages, beams, evictions -- must move each group's step and zero with its codes).

* Codes moved without their metadata decode to different keys and values, and
  the attention output changes: a remap that left the scales behind would be
  visible.
* Codes moved together with their metadata decode to exactly the moved
  reconstruction: a key block (channel axis) and a token (token axis) carry
  everything needed to decode them, so pages may sit anywhere.
* Dropping whole key blocks from a history (an eviction of whole pages)
  leaves the encoding of every other block unchanged: the encoding of the
  shortened history is the old encoding with those blocks removed.

CPU only; the oracle is the plain definition, so these are properties of the
method as the pages state it, checked on seeded inputs."""

import numpy as np
import pytest

from oracle import kvq_oracle as o

G = 32


def _history(T, D, seed):
    rng = np.random.default_rng(seed)
    k = rng.standard_normal((T, D)).astype(np.float32)
    k[:, 5] *= 20.0  # an outlier channel, as keys have ([U] "Chaves: Os Valores Extremos Vivem em Canais Fixos")
    v = rng.standard_normal((T, D)).astype(np.float32)
    return k, v


def _enc(k, v, bits_k=3, bits_v=4):
    return o.encode_head(k, v, group_k=G, group_v=G, axis_k=o.AXIS_CHANNEL, axis_v=o.AXIS_TOKEN, bits_k=bits_k,
                         bits_v=bits_v)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_codes_moved_without_metadata_change_the_output(seed):
    D, T = 64, 4 * G + 5
    k, v = _history(T, D, seed)
    e = _enc(k, v)
    q = np.random.default_rng(100 + seed).standard_normal((2, D))
    ref = o.attend(q, e["k_hat"], e["v_hat"], 1.0 / np.sqrt(D))
    perm = [2, 0, 3, 1]  # key blocks in another order
    rows = np.concatenate([np.arange(b * G, (b + 1) * G) for b in perm])
    nq = 4 * G
    # keys: block codes moved, the per-channel steps and zeros left in place
    kc = e["k_codes"][rows]
    k_bad = o.dequantize_tensor(kc, e["k_scale"], e["k_zero"], e["k_resid"], o.AXIS_CHANNEL, G)
    out = o.attend(q, k_bad, e["v_hat"], 1.0 / np.sqrt(D))
    assert np.abs(out - ref).max() > 1e-2 * np.abs(ref).max()
    # values: token codes moved, the per-token steps and zeros left in place
    vc = e["v_codes"][np.concatenate([rows, np.arange(nq, T)])]
    v_bad = o.dequantize_tensor(vc, e["v_scale"], e["v_zero"], e["v_resid"], o.AXIS_TOKEN, G)
    out = o.attend(q, e["k_hat"], v_bad, 1.0 / np.sqrt(D))
    assert np.abs(out - ref).max() > 1e-2 * np.abs(ref).max()


@pytest.mark.parametrize("seed", [0, 1])
def test_codes_moved_with_their_metadata_decode_to_the_moved_reconstruction(seed):
    D, T = 64, 4 * G
    k, v = _history(T, D, seed)
    e = _enc(k, v)
    perm = [3, 1, 0, 2]
    rows = np.concatenate([np.arange(b * G, (b + 1) * G) for b in perm])
    k_moved = o.dequantize_tensor(e["k_codes"][rows], e["k_scale"][perm], e["k_zero"][perm], e["k_resid"],
                                  o.AXIS_CHANNEL, G)
    np.testing.assert_array_equal(k_moved, e["k_hat"][rows])
    v_moved = o.dequantize_tensor(e["v_codes"][rows], e["v_scale"][rows], e["v_zero"][rows], e["v_resid"],
                                  o.AXIS_TOKEN, G)
    np.testing.assert_array_equal(v_moved, e["v_hat"][rows])


@pytest.mark.parametrize("first,count,T", [(64, 64, 300), (0, 128, 260), (128, 32, 161), (32, 96, 128)])
def test_dropping_whole_blocks_keeps_every_other_encoding(first, count, T):
    D = 64
    k, v = _history(T, D, 7)
    keep = np.concatenate([np.arange(0, first), np.arange(first + count, T)])
    full, cut = _enc(k, v), _enc(k[keep], v[keep])
    nb0, nb = first // G, count // G
    kept_blocks = [b for b in range(len(full["k_scale"])) if not nb0 <= b < nb0 + nb]
    np.testing.assert_array_equal(cut["k_meta"], full["k_meta"][kept_blocks])
    kept_rows = np.concatenate([np.arange(b * G, (b + 1) * G) for b in kept_blocks]) if kept_blocks else \
        np.zeros(0, np.int64)
    np.testing.assert_array_equal(cut["k_words"], full["k_words"][kept_rows])
    np.testing.assert_array_equal(cut["k_resid"], full["k_resid"])
    np.testing.assert_array_equal(cut["v_words"], full["v_words"][keep])
    np.testing.assert_array_equal(cut["v_meta"], full["v_meta"][keep])
    np.testing.assert_array_equal(cut["k_hat"], full["k_hat"][keep])
