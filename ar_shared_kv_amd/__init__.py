"""Orthrus decode-step hot path for MI355X (gfx950).

The product is the C-ABI library ``liborthrus.so`` (include/orthrus.h):
shared-KV block attention (orthrus_block_attn), exact consensus
(orthrus_consensus, orthrus_argmax) and the compacting KV append
(orthrus_kv_append).  ``ar_shared_kv_amd._binding`` is its ctypes binding
and ``ar_shared_kv_amd.api`` a tensor-level convenience layer.  Submodules
load lazily so that building does not need the library.
"""

__all__ = ["api", "_binding", "build"]


def __getattr__(name):
    import importlib
    if name in __all__:
        return importlib.import_module(f"{__name__}.{name}")
    raise AttributeError(name)
