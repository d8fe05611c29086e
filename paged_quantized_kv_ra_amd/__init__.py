"""paged_quantized_kv_ra_amd: paged, quantized-KV decode/verify attention for MI355X.

The compute lives in ``libra_kv.so`` (hand-written HIP for gfx950, C ABI in
``include/ra_kv.h``).  This package only marshals arguments into it; the
library is loaded on first use and a missing or unloadable library raises
at once (there is no fallback).
"""

__all__ = ["kv_store", "paged_attn", "lse_merge", "kv_gather_dequant",
           "paged_attn_workspace", "abi_version", "load_library", "new_cache", "new_scale_plane", "RaError",
           "rope_table", "qkv_rope_store"]


def __getattr__(name):
    if name in __all__:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
