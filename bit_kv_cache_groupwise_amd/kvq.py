"""ctypes binding of libkvq (include/kvq.h), same call names.

Argument marshalling only: every step of quantize, append, decode attention
and dequantize runs in the library's HIP kernels. torch provides device
memory and the current stream. Importing this module raises ImportError when
libkvq.so has not been built (python -m bit_kv_cache_groupwise_amd.build).
"""

from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
# KVQ_LIBRARY selects another build of the same library (benchmarking variants).
LIB_PATH = os.environ.get("KVQ_LIBRARY") or os.path.join(_HERE, "libkvq.so")
if not os.path.exists(LIB_PATH):
    raise ImportError(f"{LIB_PATH} is missing: build it with `python -m bit_kv_cache_groupwise_amd.build`")
_lib = ctypes.CDLL(LIB_PATH)

KVQ_OK = 0
KVQ_ERR_ARG = -1
KVQ_ERR_UNSUPPORTED = -2
KVQ_ERR_CAPACITY = -3
KVQ_ERR_ALIGN = -4
KVQ_ERR_WORKSPACE = -5
KVQ_ERR_HIP = -6

KVQ_AXIS_CHANNEL = 0
KVQ_AXIS_TOKEN = 1
KVQ_F32, KVQ_F16, KVQ_BF16 = 0, 1, 2
KVQ_DECODE_SINGLE_QUERY, KVQ_DECODE_QUERY_GROUP, KVQ_DECODE_GENERIC = 1, 2, 3
DTYPE_CODE = {"f32": KVQ_F32, "f16": KVQ_F16, "bf16": KVQ_BF16}

EXPORTED = ("kvq_plan", "kvq_cache_create", "kvq_cache_destroy", "kvq_quantize_append",
            "kvq_decode_workspace_size", "kvq_decode_attention", "kvq_dequantize", "kvq_seq_lengths",
            "kvq_get_region", "kvq_status_string", "kvq_last_error", "kvq_version", "kvq_read_probe", "kvq_decode_attention_layers",
            "kvq_quantize_append_layers", "kvq_decode_step", "kvq_copy_sequence", "kvq_decode_attention_noalloc",
            "kvq_gather_sequences", "kvq_evict_tokens", "kvq_reset_sequence", "kvq_page_list", "kvq_decode_kernel")


class kvq_geometry(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "layers", "num_seqs", "kv_heads", "q_heads", "head_dim", "group_k", "group_v",
        "axis_k", "axis_v", "in_dtype", "meta_dtype", "window", "sinks")] + [("rope_base", ctypes.c_double)] + [
        (n, ctypes.c_int32) for n in ("page_tokens", "num_pages")]


class kvq_sizes(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "codes_bytes", "meta_bytes", "residual_bytes", "table_bytes",
        "formula_codes_bytes", "formula_meta_bytes", "formula_residual_bytes", "page_bytes", "num_pages")]


class kvq_region(ctypes.Structure):
    _fields_ = [(n, ctypes.c_uint64) for n in (
        "k_codes", "v_codes", "k_meta", "v_meta", "k_resid", "v_resid",
        "k_codes_head_stride", "v_codes_head_stride", "k_meta_head_stride", "v_meta_head_stride",
        "k_resid_head_stride", "v_resid_head_stride")] + [
        (n, ctypes.c_int32) for n in ("bits_k", "bits_v", "capacity", "length")]


_P = ctypes.c_void_p
_I32P = ctypes.POINTER(ctypes.c_int32)
_U8P = ctypes.POINTER(ctypes.c_uint8)

_lib.kvq_plan.argtypes = [ctypes.POINTER(kvq_geometry), _I32P, _U8P, _U8P, ctypes.POINTER(kvq_sizes)]
_lib.kvq_cache_create.argtypes = [ctypes.POINTER(kvq_geometry), _I32P, _U8P, _U8P, _P, _P, _P, _P, _P,
                                  ctypes.POINTER(_P)]
_lib.kvq_cache_destroy.argtypes = [_P]
_lib.kvq_cache_destroy.restype = None
_lib.kvq_quantize_append.argtypes = [_P, ctypes.c_int32, _P, _P, _I32P, _P]
_lib.kvq_copy_sequence.argtypes = [_P, ctypes.c_int32, _P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]
_lib.kvq_quantize_append_layers.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _P, _P, _I32P, _P]
_lib.kvq_decode_step.argtypes = [_P, ctypes.c_int32, _P, _P, _I32P, _P, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
_lib.kvq_decode_kernel.argtypes = [_P, _I32P]
_lib.kvq_decode_workspace_size.argtypes = [_P]
_lib.kvq_decode_workspace_size.restype = ctypes.c_size_t
_lib.kvq_decode_attention.argtypes = [_P, ctypes.c_int32, _P, ctypes.c_float, _P, _P, ctypes.c_size_t, _P]
_lib.kvq_decode_attention_noalloc.argtypes = [_P, ctypes.c_int32, _P, ctypes.c_float, _P, _P]
_lib.kvq_decode_attention_layers.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _P, ctypes.c_float, _P, _P,
                                             ctypes.c_size_t, _P]
_lib.kvq_dequantize.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _P, _P, _P]
_lib.kvq_seq_lengths.argtypes = [_P, ctypes.c_int32, _I32P]
_lib.kvq_gather_sequences.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, _I32P, _P]
_lib.kvq_evict_tokens.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                  _P]
_lib.kvq_reset_sequence.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32, _P]
_lib.kvq_page_list.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_uint32), ctypes.c_int32,
                               _I32P, ctypes.POINTER(ctypes.c_int64)]
_lib.kvq_read_probe.argtypes = [_P, ctypes.c_uint64, _P, _P]
_lib.kvq_get_region.argtypes = [_P, ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(kvq_region)]
_lib.kvq_status_string.argtypes = [ctypes.c_int32]
_lib.kvq_status_string.restype = ctypes.c_char_p
_lib.kvq_last_error.argtypes = []
_lib.kvq_last_error.restype = ctypes.c_char_p
_lib.kvq_version.argtypes = []
_lib.kvq_version.restype = ctypes.c_char_p
for _n in ("kvq_plan", "kvq_cache_create", "kvq_quantize_append", "kvq_decode_attention", "kvq_dequantize",
           "kvq_seq_lengths", "kvq_get_region", "kvq_read_probe", "kvq_decode_attention_layers",
            "kvq_quantize_append_layers", "kvq_decode_step", "kvq_copy_sequence", "kvq_decode_attention_noalloc",
           "kvq_gather_sequences", "kvq_evict_tokens", "kvq_reset_sequence", "kvq_page_list"):
    getattr(_lib, _n).restype = ctypes.c_int32


class KVQError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        msg = _lib.kvq_last_error().decode()
        super().__init__(f"{call}: {_lib.kvq_status_string(status).decode()} ({status}): {msg}")


def _check(status: int, call: str):
    if status != KVQ_OK:
        raise KVQError(status, call)


def _i32(seq):
    if isinstance(seq, ctypes.Array):  # already marshalled (hot loops build it once)
        return seq
    return (ctypes.c_int32 * len(seq))(*[int(v) for v in seq])


def _u8(seq):
    return (ctypes.c_uint8 * len(seq))(*[int(v) for v in seq])


def _ptr(t) -> int:
    return 0 if t is None else (t if isinstance(t, int) else t.data_ptr())


def _stream(stream):
    if stream is None:
        import torch
        return torch.cuda.current_stream().cuda_stream
    return stream if isinstance(stream, int) else stream.cuda_stream


def geometry(*, layers, num_seqs, kv_heads, q_heads, head_dim, group_k, group_v,
             axis_k=KVQ_AXIS_CHANNEL, axis_v=KVQ_AXIS_TOKEN, in_dtype="f16", meta_dtype=KVQ_F16,
             window=0, sinks=0, rope_base=0.0, page_tokens=0, num_pages=0):
    return kvq_geometry(layers, num_seqs, kv_heads, q_heads, head_dim, group_k, group_v, axis_k, axis_v,
                        DTYPE_CODE.get(in_dtype, in_dtype), meta_dtype, window, sinks, float(rope_base),
                        page_tokens, num_pages)


# ---------------------------------------------------------------------------
# The C calls, one to one
# ---------------------------------------------------------------------------

def kvq_status_string(status: int) -> str:
    return _lib.kvq_status_string(status).decode()


def kvq_last_error() -> str:
    return _lib.kvq_last_error().decode()


def kvq_version() -> str:
    return _lib.kvq_version().decode()


def kvq_plan(geom: kvq_geometry, capacity, bits_k, bits_v) -> kvq_sizes:
    out = kvq_sizes()
    _check(_lib.kvq_plan(ctypes.byref(geom), _i32(capacity), _u8(bits_k), _u8(bits_v), ctypes.byref(out)), "kvq_plan")
    return out


def kvq_plan_status(geom, capacity, bits_k, bits_v) -> int:
    """Raw status of kvq_plan (for error-path tests)."""
    out = kvq_sizes()
    cap = _i32(capacity) if capacity is not None else None
    bk = _u8(bits_k) if bits_k is not None else None
    bv = _u8(bits_v) if bits_v is not None else None
    return _lib.kvq_plan(ctypes.byref(geom) if geom is not None else None, cap, bk, bv, ctypes.byref(out))


def kvq_cache_create(geom, capacity, bits_k, bits_v, d_codes, d_meta, d_residual, d_table, stream=None) -> int:
    h = _P()
    _check(_lib.kvq_cache_create(ctypes.byref(geom), _i32(capacity), _u8(bits_k), _u8(bits_v), _ptr(d_codes),
                                 _ptr(d_meta), _ptr(d_residual), _ptr(d_table), _stream(stream), ctypes.byref(h)),
           "kvq_cache_create")
    return h.value


def kvq_cache_create_status(geom, capacity, bits_k, bits_v, d_codes, d_meta, d_residual, d_table, stream=0) -> int:
    """Raw status of kvq_cache_create (for error-path tests); destroys a created handle."""
    h = _P()
    st = _lib.kvq_cache_create(ctypes.byref(geom), _i32(capacity), _u8(bits_k), _u8(bits_v), _ptr(d_codes),
                               _ptr(d_meta), _ptr(d_residual), _ptr(d_table), stream, ctypes.byref(h))
    if h.value:
        _lib.kvq_cache_destroy(h.value)
    return st


def kvq_cache_destroy(handle: int):
    _lib.kvq_cache_destroy(handle)


def kvq_quantize_append(handle, layer, k_new, v_new, n_new, stream=None):
    _check(_lib.kvq_quantize_append(handle, layer, _ptr(k_new), _ptr(v_new), _i32(n_new), _stream(stream)),
           "kvq_quantize_append")


def kvq_quantize_append_layers(handle, layer0, n_layers, k_new, v_new, n_new, stream=None):
    _check(_lib.kvq_quantize_append_layers(handle, layer0, n_layers, _ptr(k_new), _ptr(v_new), _i32(n_new),
                                           _stream(stream)), "kvq_quantize_append_layers")


def kvq_decode_step(handle, layer, k_new, v_new, n_new, q, softmax_scale, out, workspace, workspace_bytes=None,
                    stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.kvq_decode_step(handle, layer, _ptr(k_new), _ptr(v_new), _i32(n_new), _ptr(q),
                                ctypes.c_float(softmax_scale), _ptr(out), _ptr(workspace), workspace_bytes,
                                _stream(stream)), "kvq_decode_step")


def kvq_decode_kernel(handle) -> int:
    """KVQ_DECODE_SINGLE_QUERY, KVQ_DECODE_QUERY_GROUP or KVQ_DECODE_GENERIC."""
    out = (ctypes.c_int32 * 1)()
    _check(_lib.kvq_decode_kernel(handle, out), "kvq_decode_kernel")
    return int(out[0])


def kvq_decode_workspace_size(handle) -> int:
    return int(_lib.kvq_decode_workspace_size(handle))


def kvq_decode_attention(handle, layer, q, softmax_scale, out, workspace, workspace_bytes=None, stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.kvq_decode_attention(handle, layer, _ptr(q), ctypes.c_float(softmax_scale), _ptr(out),
                                     _ptr(workspace), workspace_bytes, _stream(stream)), "kvq_decode_attention")


def kvq_decode_attention_noalloc(handle, layer, q, softmax_scale, out, stream=None):
    _check(_lib.kvq_decode_attention_noalloc(handle, layer, _ptr(q), ctypes.c_float(softmax_scale), _ptr(out),
                                             _stream(stream)), "kvq_decode_attention_noalloc")


def kvq_decode_attention_layers(handle, layer0, n_layers, q, softmax_scale, out, workspace, workspace_bytes=None,
                                stream=None):
    if workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check(_lib.kvq_decode_attention_layers(handle, layer0, n_layers, _ptr(q), ctypes.c_float(softmax_scale),
                                            _ptr(out), _ptr(workspace), workspace_bytes, _stream(stream)),
           "kvq_decode_attention_layers")


def kvq_copy_sequence(dst_handle, dst_seq, src_handle, src_seq, layer0, n_layers, stream=None):
    _check(_lib.kvq_copy_sequence(dst_handle, dst_seq, src_handle, src_seq, layer0, n_layers, _stream(stream)),
           "kvq_copy_sequence")


def kvq_gather_sequences(handle, layer0, n_layers, src, stream=None):
    _check(_lib.kvq_gather_sequences(handle, layer0, n_layers, _i32(src), _stream(stream)), "kvq_gather_sequences")


def kvq_evict_tokens(handle, layer0, n_layers, seq, first, count, stream=None):
    _check(_lib.kvq_evict_tokens(handle, layer0, n_layers, seq, first, count, _stream(stream)), "kvq_evict_tokens")


def kvq_reset_sequence(handle, layer0, n_layers, seq, stream=None):
    _check(_lib.kvq_reset_sequence(handle, layer0, n_layers, seq, _stream(stream)), "kvq_reset_sequence")


def kvq_page_list(handle, layer, seq):
    """(physical page of each logical page, free pages of the pool)."""
    n = ctypes.c_int32()
    free = ctypes.c_int64()
    _check(_lib.kvq_page_list(handle, layer, seq, None, 0, ctypes.byref(n), ctypes.byref(free)), "kvq_page_list")
    out = (ctypes.c_uint32 * max(1, n.value))()
    _check(_lib.kvq_page_list(handle, layer, seq, out, n.value, ctypes.byref(n), ctypes.byref(free)), "kvq_page_list")
    return list(out)[:n.value], free.value


def kvq_read_probe(buf, nbytes, sink, stream=None):
    """Streaming read of nbytes of device memory at buf (measurement aid)."""
    _check(_lib.kvq_read_probe(_ptr(buf), nbytes, _ptr(sink), _stream(stream)), "kvq_read_probe")


def kvq_dequantize(handle, layer, seq, k_out, v_out, stream=None):
    _check(_lib.kvq_dequantize(handle, layer, seq, _ptr(k_out), _ptr(v_out), _stream(stream)), "kvq_dequantize")


def kvq_seq_lengths(handle, layer, num_seqs):
    out = (ctypes.c_int32 * num_seqs)()
    _check(_lib.kvq_seq_lengths(handle, layer, out), "kvq_seq_lengths")
    return list(out)


def kvq_get_region(handle, layer, seq) -> kvq_region:
    out = kvq_region()
    _check(_lib.kvq_get_region(handle, layer, seq, ctypes.byref(out)), "kvq_get_region")
    return out


def raw():
    """The ctypes library object (for calls with hand-made arguments in tests)."""
    return _lib


# ---------------------------------------------------------------------------
# Holder of the torch-allocated pools of one cache (marshalling only)
# ---------------------------------------------------------------------------

class Cache:
    """Owns the four device pools (torch uint8 tensors) and the library handle."""

    def __init__(self, geom: kvq_geometry, capacity, bits_k, bits_v, device="cuda"):
        import torch
        self.geom = geom
        self.capacity = [int(c) for c in capacity]
        self.bits_k = [int(b) for b in bits_k]
        self.bits_v = [int(b) for b in bits_v]
        self.sizes = kvq_plan(geom, self.capacity, self.bits_k, self.bits_v)
        mk = lambda n: torch.empty(int(n), dtype=torch.uint8, device=device)
        self.codes = mk(self.sizes.codes_bytes)
        self.meta = mk(self.sizes.meta_bytes)
        self.resid = mk(self.sizes.residual_bytes)
        self.table = mk(self.sizes.table_bytes)
        for t in (self.codes, self.meta, self.resid, self.table):
            if t.data_ptr() % 256:
                raise RuntimeError("torch returned a device block that is not 256-byte aligned")
        self.handle = kvq_cache_create(geom, self.capacity, self.bits_k, self.bits_v,
                                       self.codes, self.meta, self.resid, self.table)
        self._ws = None

    def close(self):
        if self.handle:
            kvq_cache_destroy(self.handle)
            self.handle = 0

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass

    def append(self, layer, k_new, v_new, n_new, stream=None):
        kvq_quantize_append(self.handle, layer, k_new, v_new, n_new, stream)

    def append_layers(self, layer0, k_new, v_new, n_new, stream=None):
        """Append into layers [layer0, layer0 + len(k_new)); k_new, v_new:
        [n_layers][sum n_new][kv_heads][head_dim]."""
        kvq_quantize_append_layers(self.handle, layer0, int(k_new.shape[0]), k_new, v_new, n_new, stream)

    def workspace(self, n_layers=1):
        """Decode workspace for calls covering up to n_layers layers (grown on demand)."""
        import torch
        need = n_layers * kvq_decode_workspace_size(self.handle)
        if self._ws is None or self._ws.numel() < need:
            self._ws = torch.empty(need, dtype=torch.uint8, device=self.codes.device)
        return self._ws

    def decode(self, layer, q, softmax_scale, out=None, stream=None):
        import torch
        g = self.geom
        if out is None:
            out = torch.empty((g.num_seqs, g.q_heads, g.head_dim), dtype=torch.float32, device=q.device)
        ws = self.workspace()
        kvq_decode_attention(self.handle, layer, q, softmax_scale, out, ws, ws.numel(), stream)
        return out

    def step(self, layer, k_new, v_new, n_new, q, softmax_scale, out=None, stream=None):
        """Append the new rows and attend (one decode step of one layer)."""
        import torch
        g = self.geom
        if out is None:
            out = torch.empty((g.num_seqs, g.q_heads, g.head_dim), dtype=torch.float32, device=q.device)
        ws = self.workspace()
        kvq_decode_step(self.handle, layer, k_new, v_new, n_new, q, softmax_scale, out, ws, ws.numel(), stream)
        return out

    def decode_layers(self, layer0, n_layers, q, softmax_scale, out=None, stream=None):
        """Decode attention of layers [layer0, layer0 + n_layers) in one call;
        q: [n_layers][num_seqs][q_heads][head_dim]."""
        import torch
        g = self.geom
        if out is None:
            out = torch.empty((n_layers, g.num_seqs, g.q_heads, g.head_dim), dtype=torch.float32, device=q.device)
        ws = self.workspace(n_layers)
        kvq_decode_attention_layers(self.handle, layer0, n_layers, q, softmax_scale, out, ws, ws.numel(), stream)
        return out

    def dequantize(self, layer, seq, stream=None):
        import torch
        g = self.geom
        n = self.lengths(layer)[seq]
        k = torch.empty((g.kv_heads, n, g.head_dim), dtype=torch.float32, device=self.codes.device)
        v = torch.empty_like(k)
        kvq_dequantize(self.handle, layer, seq, k, v, stream)
        return k, v

    def copy_sequence(self, dst_seq, src_cache, src_seq, layer0=0, n_layers=None, stream=None):
        n = self.geom.layers - layer0 if n_layers is None else n_layers
        kvq_copy_sequence(self.handle, dst_seq, src_cache.handle, src_seq, layer0, n, stream)

    def gather(self, src, layer0=0, n_layers=None, stream=None):
        """Sequence s takes what sequence src[s] held (beam reorder, forks)."""
        n = self.geom.layers - layer0 if n_layers is None else n_layers
        kvq_gather_sequences(self.handle, layer0, n, src, stream)

    def evict(self, seq, first, count, layer0=0, n_layers=None, stream=None):
        n = self.geom.layers - layer0 if n_layers is None else n_layers
        kvq_evict_tokens(self.handle, layer0, n, seq, first, count, stream)

    def reset(self, seq, layer0=0, n_layers=None, stream=None):
        n = self.geom.layers - layer0 if n_layers is None else n_layers
        kvq_reset_sequence(self.handle, layer0, n, seq, stream)

    def page_list(self, layer, seq):
        return kvq_page_list(self.handle, layer, seq)

    def decode_kernel(self):
        return kvq_decode_kernel(self.handle)

    def lengths(self, layer):
        return kvq_seq_lengths(self.handle, layer, self.geom.num_seqs)

    def region(self, layer, seq) -> kvq_region:
        return kvq_get_region(self.handle, layer, seq)
