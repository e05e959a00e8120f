"""kvq_decode_attention_noalloc, the decode call for callers that cannot
allocate device memory (its split workspace is the library's fixed device
array), against kvq_decode_attention with a caller-owned workspace, through the
C ABI: identical outputs bit for bit on two calls in a row (the second on a
smaller cache, so the array holds the first call's partials), both within the
oracle's row tolerance, and the limit error before anything is written."""

import sys

import numpy as np
import pytest
import torch

from bit_kv_cache_groupwise_amd import workloads as W
from tests import gpu_helpers as H

pytestmark = pytest.mark.gpu


def _note(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def _filled(w, **kw):
    cache = H.make_cache(w, **kw)
    prefix, new = H.history(w, 0)
    cache.append(0, prefix[0].cuda(), prefix[1].cuda(), prefix[2])
    cache.append(0, new[0].cuda(), new[1].cuda(), new[2])
    torch.cuda.synchronize()
    return cache, prefix, new


def test_noalloc_equals_workspace_call_on_two_calls():
    kvq = H.kvq()
    big = W.mixed_batch().scaled(num_seqs=8, lengths=(9000, 700, 33, 20000, 4096, 1, 12000, 300))
    small = W.llama2_7b().scaled(num_seqs=3, kv_heads=4, q_heads=4, lengths=(1000, 50, 2))
    for w in (big, small):
        _note(f"[noalloc] S={w.num_seqs} Hq={w.q_heads} Hkv={w.kv_heads} D={w.head_dim} lens={w.lengths}")
        cache, prefix, new = _filled(w)
        q = W.draw_q(w, 0).cuda()
        ref = cache.decode(0, q, w.softmax_scale)
        out = torch.full_like(ref, float("nan"))
        kvq.kvq_decode_attention_noalloc(cache.handle, 0, q, w.softmax_scale, out)
        torch.cuda.synchronize()
        assert torch.equal(out, ref), w.lengths
        got = out.cpu().numpy()
        for s in (0, w.num_seqs - 1):
            k, v = H.full_seq(prefix, new, s)
            encs = [H.encode(w, k, v, s, h) for h in range(w.kv_heads)]
            err = H.row_rel_err(got[s], H.attn_ref(w, q[s].float().cpu().numpy(), encs))
            assert np.all(err <= H.ATTN_TOL), (s, float(err.max()))
        cache.close()


def test_noalloc_rejects_a_workspace_beyond_the_fixed_array():
    """A call whose split workspace exceeds the fixed 64 MiB array (here the
    slots of a 4000-token full-precision window for 128 query heads) fails with
    KVQ_ERR_WORKSPACE and writes nothing; the workspace call still works."""
    kvq = H.kvq()
    w = W.long_gqa().scaled(num_seqs=16, kv_heads=4, q_heads=128, lengths=(40,) * 16, bits=((4, 8),) * 16)
    cache, _, _ = _filled(w, window=4000)
    q = W.draw_q(w, 0).cuda()
    out = torch.full((w.num_seqs, w.q_heads, w.head_dim), float("nan"), device="cuda")
    with pytest.raises(kvq.KVQError) as e:
        kvq.kvq_decode_attention_noalloc(cache.handle, 0, q, w.softmax_scale, out)
    assert e.value.status == kvq.KVQ_ERR_WORKSPACE
    assert "fixed scratch" in str(e.value)
    torch.cuda.synchronize()
    assert torch.isnan(out).all()
    ref = cache.decode(0, q, w.softmax_scale)
    torch.cuda.synchronize()
    assert torch.isfinite(ref).all()
    cache.close()
