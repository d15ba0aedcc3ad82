"""MI355X-native MLA decode: latent-space attention over a compressed KV cache.

The compute lives in ``libmla.so`` (hand-written HIP kernels for gfx950 behind
a C ABI declared in ``include/mla.h``).  The functions here marshal torch
tensors to that ABI; they load the library on first use and raise if it is
missing.  ``inputs`` (seeded synthetic workloads) imports nothing from here.
"""

__all__ = ["absorb_q", "append_cache", "decode_attn", "decode_attn_causal", "project_out",
           "cache_row_bytes", "decode_attn_workspace", "decode_attn_causal_workspace", "Dims",
           "MLAError", "lib", "absorb_q_normed", "append_cache_normed"]


def __getattr__(name):
    if name in __all__:
        from . import _lib
        return getattr(_lib, name)
    raise AttributeError(name)
