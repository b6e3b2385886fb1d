"""MI355X-native attention over a per-layer KV cache.

The compute path is ``libkvcache.so``: hand-written HIP kernels for gfx950
behind a C ABI (``include/kvcache.h``).  ``transformer_kv_cache_amd.kvcache``
is the thin ctypes binding over it; ``synth`` makes seeded synthetic inputs.
The binding is imported lazily so that input generation works without a GPU.
"""
__all__ = ["kvcache", "synth"]


def __getattr__(name):
    if name in __all__:
        import importlib
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
