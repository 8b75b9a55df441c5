"""Paged-KV-cache decode attention for MI355X (gfx950).

The compute lives in ``libpa.so`` (hand-written HIP kernels behind a C ABI,
declared in ``include/pa.h``). ``paged_kv_cache_380_amd.binding`` marshals
torch tensors into that ABI; importing this package does not load the library,
so the CPU-only parts (``workloads``) stay importable without it. Calling an
operation when the library is missing raises ``RuntimeError``.
"""

__all__ = ["binding", "workloads"]


def __getattr__(name):
    if name in ("reshape_and_cache", "decode", "decode_workspace_bytes"):
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
