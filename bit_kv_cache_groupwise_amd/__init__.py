"""Groupwise bit-packed KV-cache quantization with fused decode attention on
AMD Instinct MI355X (gfx950).

The compute lives in ``libkvq.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/kvq.h``); ``kvq`` is a thin ctypes binding with the same
call names. Importing the binding fails loudly if the library is not built.
"""

from . import workloads  # noqa: F401  (input generators; no method arithmetic)


def lib():
    """The loaded ctypes binding (raises if libkvq.so is missing)."""
    from . import kvq
    return kvq
