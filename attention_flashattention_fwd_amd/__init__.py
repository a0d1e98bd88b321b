"""MI355X-native attention hot path: hand-written gfx950 HIP kernels behind a
C-ABI library (forward, continuation over a KV cache, paged decode, backward,
fused RMSNorm).

The entry points live in `binding` and are imported lazily, so that the
CPU-only pieces (the seeded input generators) load without the HIP library.
"""

__all__ = ["attn_fwd", "attn_fwd_into", "attn_fwd_kv", "attn_fwd_kv_into", "attn_bwd",
           "paged_decode", "paged_decode_into", "paged_workspace_bytes", "rmsnorm_fwd",
           "rmsnorm_fwd_into", "library_path", "version"]


def __getattr__(name):
    if name in __all__:
        from . import binding
        return getattr(binding, name)
    raise AttributeError(name)
