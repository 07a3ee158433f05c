"""windowed_attention_amd: chunk-causal rolling-KV attention for MI355X (gfx950).

The compute lives in libuf.so (hand-written HIP kernels behind the C ABI of
include/uf.h); `uf` is its ctypes binding.  Using the binding requires the
built library: there is no other code path, and the first access to `uf`,
`KVCache` or `UfError` raises ImportError when libuf.so is missing.  The
`build` submodule imports without the library, so that it can build it.
"""
import importlib

__all__ = ["uf", "KVCache", "UfError"]


def __getattr__(name):
    if name in __all__:
        uf = importlib.import_module(".uf", __name__)
        return uf if name == "uf" else getattr(uf, name)
    raise AttributeError(f"module {__name__!r} has no attribute {name!r}")
