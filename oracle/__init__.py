"""fp64 CPU oracle for the attention path (test infrastructure only).

Only the tests, the package smoke check and the bench's CPU-baseline leg may
import this package.  The HIP library never uses it.
"""
from .oracle import (  # noqa: F401
    OracleLib,
    attn_bwd,
    attn_bwd_rows,
    attn_fwd,
    attn_fwd_kv,
    attn_probs,
    attn_rows,
    build,
    load,
    paged_decode,
    rmsnorm,
    threads,
)
