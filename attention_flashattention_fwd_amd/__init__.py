"""MI355X-native FlashAttention-style forward pass for causal grouped-query
attention: hand-written gfx950 HIP kernels behind a C-ABI library.

`attn_fwd` and friends live in `binding` and are imported lazily so that the
CPU-only pieces (the seeded input generator) load without the HIP library.
"""

__all__ = ["attn_fwd", "attn_fwd_into", "library_path", "version"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
