"""The benchmark's algorithmic byte counts (CPU): without a window, the size
formula of one (layer, seq, kv head) ([N] "Ukuran cache bertambah ..."); with a
full-precision window and sinks, the codes and (step, zero) pairs of the tokens
the oracle reads quantized plus both tensors' rows of the tokens it reads
exactly."""

import numpy as np
import pytest

import bench
from oracle import kvq_oracle as o


@pytest.mark.parametrize("T", [0, 1, 31, 32, 33, 100, 4097])
@pytest.mark.parametrize("bk,bv", [(2, 2), (6, 4), (4, 8)])
def test_plain_bytes_equal_the_size_formula(T, bk, bv):
    hb = o.head_bytes(T, 128, group_k=32, group_v=32, axis_k=o.AXIS_CHANNEL, axis_v=o.AXIS_TOKEN, bits_k=bk,
                      bits_v=bv, in_bytes=2)
    assert bench.algorithmic_head_bytes(T, 128, 0, 1, 32, 32, bk, bv, 2) == hb["total"]


@pytest.mark.parametrize("T", [1, 20, 150, 161, 4097, 262145])
@pytest.mark.parametrize("window,sinks", [(128, 32), (0, 64), (50, 0)])
def test_window_bytes_follow_the_oracle_mask(T, window, sinks):
    D, G, ib = 128, 32, 2
    mask = o.full_precision_mask(T, window, sinks, G)
    nq = int((~mask).sum())
    assert nq % G == 0
    expect = 2 * (T - nq) * D * ib + nq * D * (2 + 4) // 8 + (nq // G) * D * 4 + nq * (D // G) * 4
    assert bench.algorithmic_head_bytes(T, D, 0, 1, G, G, 2, 4, ib, window=window, sinks=sinks) == expect
