"""windowed_attention_amd: chunk-causal rolling-KV attention for MI355X (gfx950).

The compute lives in libuf.so (hand-written HIP kernels behind the C ABI of
include/uf.h); `uf` is its ctypes binding.  Importing the binding requires
the built library: there is no other code path.
"""
from . import uf
from .uf import KVCache, UfError

__all__ = ["uf", "KVCache", "UfError"]
