"""Batched attention over a paged KV cache on AMD Instinct MI355X (gfx950).

The compute path is libpkv.so (include/pkv.h): a host C++ planner and HIP
kernels for decode (split-KV + merge), prefill (bf16 MFMA), the mixed step and
KV append.  `pkv` is the ctypes binding; `wrappers` holds plan/run classes
shaped like the mstar attn.wrappers page.  Importing either requires the built
library; there is no fallback path.
"""
__all__ = ["pkv", "wrappers", "DecodeWrapper", "PrefillWrapper", "MixedWrapper"]


def __getattr__(name):
    if name in ("pkv", "wrappers"):
        import importlib
        return importlib.import_module(f".{name}", __name__)
    if name in ("DecodeWrapper", "PrefillWrapper", "MixedWrapper"):
        from . import wrappers
        return getattr(wrappers, name)
    raise AttributeError(name)
