"""kvsel for MI355X: query-aware sparse-page decode attention over a paged GQA KV cache.

Every step of the path runs in hand-written HIP kernels for gfx950 behind the C ABI declared in
``include/kvsel.h`` (``libkvsel.so``); this package is the thin ctypes binding plus byte
accounting. Importing it does not load the library; the first call does, and raises if the
library has not been built.
"""
from .accounting import (  # noqa: F401
    kv_cache_bytes,
    selected_kv_bytes,
    summary_bytes,
)

__all__ = ["kv_cache_bytes", "selected_kv_bytes", "summary_bytes"]


def __getattr__(name):
    # The binding is imported lazily so that CPU-only users (the accounting) need no HIP runtime.
    if name.startswith("__") or name in ("kvsel", "build", "accounting"):
        raise AttributeError(name)
    import importlib
    _k = importlib.import_module(__name__ + ".kvsel")
    if hasattr(_k, name):
        return getattr(_k, name)
    raise AttributeError(name)
