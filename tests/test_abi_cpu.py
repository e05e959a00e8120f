"""The C-ABI library on the CPU: it loads, exports every symbol include/kvq.h
declares, sizes pools by the closed form, and rejects bad arguments before any
HIP call is made. No kernel is launched here."""

import ctypes
import os
import re
import subprocess

import pytest

from oracle import kvq_oracle as o

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "kvq.h")

kvq = pytest.importorskip("bit_kv_cache_groupwise_amd.kvq", reason="libkvq.so not built")


def declared_symbols():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(kvq_[a-z_]+)\s*\(", text)))


def test_header_declares_the_calls():
    syms = declared_symbols()
    for name in ("kvq_quantize_append", "kvq_decode_attention", "kvq_dequantize", "kvq_plan",
                 "kvq_cache_create", "kvq_cache_destroy", "kvq_decode_workspace_size", "kvq_status_string"):
        assert name in syms
    assert sorted(kvq.EXPORTED) == syms


def test_library_exports_every_declared_symbol():
    lib = kvq.raw()
    for name in declared_symbols():
        assert hasattr(lib, name), name
    nm = subprocess.run(["nm", "-D", "--defined-only", kvq.LIB_PATH], capture_output=True, text=True).stdout
    exported = set(re.findall(r"\bT (kvq_\w+)", nm))
    assert set(declared_symbols()) <= exported


def test_status_strings_and_version():
    for st in (0, -1, -2, -3, -4, -5, -6):
        assert kvq.kvq_status_string(st)
    assert kvq.kvq_status_string(12345) == "unknown status"
    assert re.match(r"\d+\.\d+\.\d+$", kvq.kvq_version())


def _geom(**kw):
    base = dict(layers=2, num_seqs=3, kv_heads=4, q_heads=8, head_dim=128, group_k=32, group_v=32)
    base.update(kw)
    return kvq.geometry(**base)


@pytest.mark.parametrize("dt,ib", [("f32", 4), ("f16", 2), ("bf16", 2)])
def test_plan_matches_closed_form(dt, ib):
    caps = [0, 1000, 4097]
    bk, bv = [2, 6, 4], [2, 4, 8]
    g = _geom(in_dtype=dt)
    sz = kvq.kvq_plan(g, caps, bk, bv)
    codes = meta = resid = 0
    for c, k, v in zip(caps, bk, bv):
        hb = o.head_bytes(c, 128, group_k=32, group_v=32, axis_k=o.AXIS_CHANNEL, axis_v=o.AXIS_TOKEN,
                          bits_k=k, bits_v=v, in_bytes=ib)
        codes += hb["codes"]
        meta += hb["meta"]
        # the residual region is G rows per channel-axis head, whatever the length
        resid += 32 * 128 * ib
    assert sz.formula_codes_bytes == 2 * 4 * codes
    assert sz.formula_meta_bytes == 2 * 4 * meta
    assert sz.formula_residual_bytes == 2 * 4 * resid
    assert sz.codes_bytes >= sz.formula_codes_bytes and sz.codes_bytes % 256 == 0
    assert sz.meta_bytes >= sz.formula_meta_bytes and sz.residual_bytes >= sz.formula_residual_bytes
    # padding is at most 255 bytes per head region
    assert sz.codes_bytes - sz.formula_codes_bytes < 256 * 2 * 3 * 4 * 2


@pytest.mark.parametrize("window,sinks,axis_k,block", [(128, 32, 0, 32), (0, 64, 0, 32), (50, 3, 1, 1)])
def test_plan_window_area(window, sinks, axis_k, block):
    """With a window or sinks every tensor head also holds sinks + window + block
    full-precision rows; codes and metadata are those of the plain cache."""
    caps = [0, 1000, 4097]
    plain = kvq.kvq_plan(_geom(axis_k=axis_k), caps, [2, 6, 4], [2, 4, 8])
    sz = kvq.kvq_plan(_geom(axis_k=axis_k, window=window, sinks=sinks), caps, [2, 6, 4], [2, 4, 8])
    assert sz.formula_codes_bytes == plain.formula_codes_bytes
    assert sz.formula_meta_bytes == plain.formula_meta_bytes
    rows = sinks + window + block
    assert sz.formula_residual_bytes == plain.formula_residual_bytes + 2 * 3 * 2 * 4 * rows * 128 * 2
    assert sz.residual_bytes >= sz.formula_residual_bytes


@pytest.mark.parametrize("window,sinks", [(0, 16), (-1, 0), (0, -32), (4096, 0), (3000, 1088)])
def test_plan_rejects_bad_window(window, sinks):
    assert kvq.kvq_plan_status(_geom(window=window, sinks=sinks), [10] * 3, [2] * 3, [2] * 3) == kvq.KVQ_ERR_ARG
    assert kvq.kvq_last_error()


@pytest.mark.parametrize("base,status", [(0.0, 0), (10000.0, 0), (500000.0, 0), (1.0, -1), (0.5, -1), (-2.0, -1),
                                         (float("nan"), -1), (float("inf"), -1)])
def test_plan_rope_base(base, status):
    """The rotary base (a double after the int32 fields) reaches the library: a base
    in (0, 1], a negative one or a non-finite one is rejected; sizes do not depend
    on it."""
    assert kvq.kvq_plan_status(_geom(rope_base=base), [10] * 3, [2] * 3, [2] * 3) == status
    if status == 0:
        assert kvq.kvq_plan(_geom(rope_base=base), [100] * 3, [2] * 3, [2] * 3).codes_bytes == \
            kvq.kvq_plan(_geom(), [100] * 3, [2] * 3, [2] * 3).codes_bytes


def test_geometry_struct_layout():
    """The binding's geometry has the header's fields in the header's order."""
    import ctypes
    hdr = open(os.path.join(ROOT, "include", "kvq.h")).read()
    body = hdr[hdr.index("typedef struct kvq_geometry {"):hdr.index("} kvq_geometry;")]
    import re
    names = re.findall(r"^\s*(?:int32_t|double)\s+(\w+);", body, flags=re.M)
    assert [f[0] for f in kvq.kvq_geometry._fields_] == names
    assert kvq.kvq_geometry.rope_base.offset == 56 and kvq.kvq_geometry.page_tokens.offset == 64
    assert ctypes.sizeof(kvq.kvq_geometry) == 72


@pytest.mark.parametrize("kw,status", [
    (dict(page_tokens=64), 0), (dict(page_tokens=4096), 0), (dict(page_tokens=65536), 0),
    (dict(page_tokens=32), -1), (dict(page_tokens=96), -1), (dict(page_tokens=131072), -1), (dict(page_tokens=-64), -1),
    (dict(page_tokens=64, group_k=128), -1), (dict(page_tokens=128, group_k=128), 0),
    (dict(page_tokens=64, sinks=32, window=16), -1), (dict(page_tokens=64, sinks=64, window=16), 0),
    (dict(page_tokens=64, num_pages=-1), -1), (dict(page_tokens=64, num_pages=5), 0),
])
def test_plan_paged_geometry(kw, status):
    """Pages hold a power of two of at least 64 tokens, at least the key block,
    and the sinks fill whole pages."""
    assert kvq.kvq_plan_status(_geom(**kw), [100] * 3, [2] * 3, [2] * 3) == status
    if status:
        assert kvq.kvq_last_error()


def test_plan_paged_sizes():
    """Paged storage: a page holds P tokens of K and V codes of every head and
    their metadata (each head region 256-byte aligned); the page stride is the
    largest over the bit pairs; the pool holds every sequence's pages at full
    capacity unless num_pages says otherwise; the table grows by one uint32 per
    logical page; the closed-form byte counts do not change."""
    D, H, P = 128, 3, 64
    g = kvq.geometry(layers=2, num_seqs=3, kv_heads=H, q_heads=H, head_dim=D, group_k=32, group_v=32)
    gp = kvq.geometry(layers=2, num_seqs=3, kv_heads=H, q_heads=H, head_dim=D, group_k=32, group_v=32, page_tokens=P)
    cap, bk, bv = [100, 64, 1000], [2, 4, 6], [2, 8, 4]
    plain, paged = kvq.kvq_plan(g, cap, bk, bv), kvq.kvq_plan(gp, cap, bk, bv)

    def a256(x):
        return (x + 255) // 256 * 256

    def page(b_k, b_v):
        return H * (a256(P * D * b_k // 8) + a256(P * D * b_v // 8) + a256(P // 32 * D * 4) + a256(P * (D // 32) * 4))

    assert paged.page_bytes == max(page(2, 2), page(4, 8), page(6, 4))
    pages = 2 * sum((c + P - 1) // P for c in cap)
    assert paged.num_pages == pages and paged.codes_bytes == pages * paged.page_bytes
    assert paged.table_bytes >= plain.table_bytes + 4 * pages - 255
    for f in ("formula_codes_bytes", "formula_meta_bytes", "formula_residual_bytes", "residual_bytes"):
        assert getattr(paged, f) == getattr(plain, f), f
    assert plain.page_bytes == 0 and plain.num_pages == 0
    small = kvq.kvq_plan(kvq.geometry(layers=2, num_seqs=3, kv_heads=H, q_heads=H, head_dim=D, group_k=32, group_v=32,
                                      page_tokens=P, num_pages=7), cap, bk, bv)
    assert small.num_pages == 7 and small.codes_bytes == 7 * paged.page_bytes


def test_plan_gpt2_effective_bits():
    """GPT-2-shaped cache (K6/V4, per-head 64-channel groups): 5.5 stored bits per
    element at a length that is a multiple of G, as the hatterialabs.com page
    prints for this configuration."""
    g = kvq.geometry(layers=12, num_seqs=8, kv_heads=12, q_heads=12, head_dim=64, group_k=64, group_v=64)
    sz = kvq.kvq_plan(g, [1024] * 8, [6] * 8, [4] * 8)
    elems = o.cache_elements(12, 1024 * 8, 12, 64)
    bits = (sz.formula_codes_bytes + sz.formula_meta_bytes) * 8 / elems
    assert bits == 5.5


@pytest.mark.parametrize("kw,status", [
    (dict(head_dim=48), -1), (dict(head_dim=512), -1), (dict(q_heads=6), -1), (dict(group_k=16), -1),
    (dict(group_v=96), -1), (dict(axis_v=2), -1), (dict(in_dtype=7), -1), (dict(layers=0), -1),
    (dict(head_dim=64, group_v=128), -1), (dict(meta_dtype=0), -2),
])
def test_plan_rejects_bad_geometry(kw, status):
    assert kvq.kvq_plan_status(_geom(**kw), [10, 10, 10], [2, 2, 2], [2, 2, 2]) == status
    assert kvq.kvq_last_error()


@pytest.mark.parametrize("bits", [1, 5, 7, 16, 0])
def test_plan_rejects_bits(bits):
    assert kvq.kvq_plan_status(_geom(), [10, 10, 10], [2, bits, 2], [2, 2, 2]) == kvq.KVQ_ERR_ARG
    assert kvq.kvq_plan_status(_geom(), [10, 10, 10], [2, 2, 2], [bits, 2, 2]) == kvq.KVQ_ERR_ARG


def test_plan_rejects_nulls_and_negative_capacity():
    assert kvq.kvq_plan_status(None, [1, 1, 1], [2] * 3, [2] * 3) == kvq.KVQ_ERR_ARG
    assert kvq.kvq_plan_status(_geom(), None, [2] * 3, [2] * 3) == kvq.KVQ_ERR_ARG
    assert kvq.kvq_plan_status(_geom(), [1, -1, 1], [2] * 3, [2] * 3) == kvq.KVQ_ERR_ARG


def test_create_validates_before_touching_the_device():
    g = _geom()
    args = ([10, 10, 10], [2] * 3, [2] * 3)
    assert kvq.kvq_cache_create_status(g, *args, 0, 256, 256, 256) == kvq.KVQ_ERR_ARG
    assert kvq.kvq_cache_create_status(g, *args, 256, 256, 256 + 4, 256) == kvq.KVQ_ERR_ALIGN
    assert kvq.kvq_cache_create_status(_geom(group_k=7), *args, 256, 256, 256, 256) == kvq.KVQ_ERR_ARG


def test_null_handle_calls_fail_cleanly():
    lib = kvq.raw()
    assert lib.kvq_quantize_append(None, 0, None, None, None, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_decode_attention(None, 0, None, ctypes.c_float(1.0), None, None, 0, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_dequantize(None, 0, 0, None, None, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_decode_workspace_size(None) == 0
    assert lib.kvq_decode_kernel(None, None) == kvq.KVQ_ERR_ARG
    lib.kvq_cache_destroy(None)
    f = ctypes.c_float(1.0)
    assert lib.kvq_decode_step(None, 0, None, None, None, None, f, None, None, 0, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_quantize_append_layers(None, 0, 1, None, None, None, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_decode_attention_layers(None, 0, 1, None, f, None, None, 0, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_copy_sequence(None, 0, None, 1, 0, 1, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_gather_sequences(None, 0, 1, None, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_evict_tokens(None, 0, 1, 0, 0, 64, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_reset_sequence(None, 0, 1, 0, None) == kvq.KVQ_ERR_ARG
    n = ctypes.c_int32()
    assert lib.kvq_page_list(None, 0, 0, None, 0, ctypes.byref(n), None) == kvq.KVQ_ERR_ARG


def test_read_probe_validates_before_launching():
    """The measurement probe rejects NULL pointers, sizes that are not whole
    16-byte vectors and misaligned pointers without touching the device (the
    pointers below are never dereferenced)."""
    lib = kvq.raw()
    assert lib.kvq_read_probe(None, 16, 0x1000, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_read_probe(0x1000, 16, None, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_read_probe(0x1000, 24, 0x2000, None) == kvq.KVQ_ERR_ARG
    assert lib.kvq_read_probe(0x1008, 32, 0x2000, None) == kvq.KVQ_ERR_ALIGN
    assert lib.kvq_read_probe(0x1000, 32, 0x2002, None) == kvq.KVQ_ERR_ALIGN
    assert lib.kvq_read_probe(0x1000, 0, 0x2000, None) == kvq.KVQ_OK  # nothing to read: no launch
