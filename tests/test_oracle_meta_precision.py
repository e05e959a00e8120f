"""Metadata precision as a format choice ([N] "Scale menentukan sistem koordinat
kuantisasi": the precision of scale and zero point is part of the format),
measured with the CPU oracle, which stores scale and zero point as fp16 or
fp32. The library stores fp16 metadata, the precision of the workloads it is
built for; these checks pin what that choice costs.

- On the Llama-2-7B-shaped recipe (keys per channel with outlier channels,
  values per token) at 2, 4 and 8 bits, fp16 metadata moves the reconstruction
  error by well under 1% of fp32's (its rounding error is small next to half a
  step).
- A group whose range is narrow next to its offset (values in [1000, 1001])
  at 8 bits: the fp16 zero point alone can be off by 0.25 (half an fp16 ulp
  at 1000) against a half step of 0.002, and the reconstruction misses by up
  to ~70 half steps, where fp32 metadata keeps the half-step bound ([U] "O Que
  o Erro de Quantizacao E Realmente Feito"). That is the regime fp32
  metadata is for.
"""

import numpy as np
import pytest

from bit_kv_cache_groupwise_amd import workloads as W
from oracle import kvq_oracle as o


def _recon(x, axis, group, bits, meta):
    codes, s, z, resid = o.quantize_tensor(x, axis, group, bits, meta)
    return o.dequantize_tensor(codes, s, z, resid, axis, group)


def _llama_rows(seed=21, T=512):
    w = W.llama2_7b().scaled(num_seqs=1, kv_heads=1, q_heads=1, lengths=(T,), bits=((2, 2),))
    k, v = W.draw_kv(w, 0, [T], device="cpu", stream=seed)
    return k[:, 0].double().numpy().astype(np.float32), v[:, 0].double().numpy().astype(np.float32)


@pytest.mark.parametrize("bits", [2, 4, 8])
def test_fp16_metadata_costs_little_on_the_llama_recipe(bits):
    k, v = _llama_rows()
    for x, axis in ((k, o.AXIS_CHANNEL), (v, o.AXIS_TOKEN)):
        e16 = np.sqrt(np.mean((_recon(x, axis, 32, bits, "f16") - x) ** 2))
        e32 = np.sqrt(np.mean((_recon(x, axis, 32, bits, "f32") - x) ** 2))
        assert abs(e16 - e32) <= 0.01 * e32, (bits, axis, e16, e32)


def test_fp16_metadata_breaks_the_half_step_bound_for_offset_groups():
    rng = np.random.default_rng(5)
    x = (1000.0 + rng.random((32, 64))).astype(np.float32)  # per-token groups of 32 channels
    for meta, ok in (("f32", True), ("f16", False)):
        codes, s, z, resid = o.quantize_tensor(x, o.AXIS_TOKEN, 32, 8, meta)
        xh = o.dequantize_tensor(codes, s, z, resid, o.AXIS_TOKEN, 32)
        half = np.repeat(s, 32, axis=1) / 2  # the stored step of each element's group
        # float32 data: one ulp of 1000 (6.1e-5) of slack for the rounding of x_hat
        within = np.all(np.abs(xh - x) <= half * (1 + 1e-6) + 6.2e-5)
        assert within == ok, meta
