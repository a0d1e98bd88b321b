"""Seeded synthetic inputs for the attention workloads (forward, continuation,
paged decode, backward) and the RMSNorm workload.

This module only draws and casts random numbers; it holds none of the
attention arithmetic, so both the HIP path's tests and the oracle may use it.

Recipe (one reading of the workloads, stated once here):
  * generator: numpy.random.default_rng(seed), PCG64;
  * draw order: Q [B,Hq,T,D], then K [B,Hkv,T,D], then V [B,Hkv,T,D], each
    with standard_normal(dtype=float32);
  * "element" outliers: after the three draws, one uniform mask for Q and
    then one for K, each entry multiplied by 8 with probability 0.01;
  * "row" outliers: masks of shape [B,Hq,T] then [B,Hkv,T], whole D-vectors
    multiplied by 8 with probability 0.01;
  * bf16 workloads are cast from those fp32 draws with round-to-nearest-even
    (torch's cast).  Multiplying by 8 is exact in both formats.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import numpy as np
import torch

OUTLIER_PROB = 0.01
OUTLIER_FACTOR = np.float32(8.0)


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    Hq: int
    Hkv: int
    T: int
    D: int
    dtype: str            # "fp32" or "bf16"
    causal: bool
    outliers: str = ""    # "", "elements" or "rows"
    seed: int = 0

    @property
    def scale(self) -> float:
        return default_scale(self.D)

    @property
    def flops(self) -> float:
        """Causal-adjusted attention FLOPs: 4*B*Hq*T^2*D, halved if causal."""
        f = 4.0 * self.B * self.Hq * self.T * self.T * self.D
        return f / 2 if self.causal else f

    @property
    def pair_flops(self) -> float:
        """4*D per visible (query, key) pair, counted exactly."""
        pairs = self.T * (self.T + 1) / 2 if self.causal else self.T * self.T
        return 4.0 * self.B * self.Hq * self.D * pairs

    def describe(self) -> str:
        o = f", outliers={self.outliers}" if self.outliers else ""
        return (f"B={self.B} Hq={self.Hq} Hkv={self.Hkv} T={self.T} D={self.D} "
                f"{self.dtype} causal={int(self.causal)}{o}")


# The five workloads of the attention forward pass, plus the two variants run
# on the same tensors (non-causal T=2048, and whole-row outliers at T=4096).
WORKLOADS = {
    "fp32_t64": Workload("fp32_t64", 1, 4, 2, 64, 32, "fp32", True),
    "tiny_t128": Workload("tiny_t128", 2, 8, 2, 128, 32, "bf16", True),
    "t2048": Workload("t2048", 8, 8, 2, 2048, 64, "bf16", True),
    "t2048_full": Workload("t2048_full", 8, 8, 2, 2048, 64, "bf16", False),
    "t4096_outliers": Workload("t4096_outliers", 16, 16, 4, 4096, 64, "bf16", True, "elements"),
    "t4096_outlier_rows": Workload("t4096_outlier_rows", 16, 16, 4, 4096, 64, "bf16", True, "rows"),
    "t16384_d128": Workload("t16384_d128", 1, 32, 8, 16384, 128, "bf16", True),
}


@dataclass(frozen=True)
class KVWorkload:
    """Tq new query rows against Tk cached key rows (tessera_attn_fwd_kv).  The
    tensors are the last Tq query rows of the full T = Tk workload drawn with
    the same recipe, so every output row is also a row of that full forward."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Tq: int
    Tk: int
    D: int
    dtype: str = "bf16"
    causal: bool = True
    seed: int = 0

    @property
    def scale(self) -> float:
        return default_scale(self.D)

    @property
    def pairs(self) -> float:
        """Visible (query, key) pairs per head: row i sees i + Tk - Tq + 1 keys."""
        if not self.causal:
            return float(self.Tq) * self.Tk
        off = self.Tk - self.Tq
        return float(self.Tq) * off + self.Tq * (self.Tq + 1) / 2

    @property
    def flops(self) -> float:
        """4*D per visible pair, counted exactly."""
        return 4.0 * self.B * self.Hq * self.D * self.pairs

    def describe(self) -> str:
        return (f"B={self.B} Hq={self.Hq} Hkv={self.Hkv} Tq={self.Tq} Tk={self.Tk} D={self.D} "
                f"{self.dtype} causal={int(self.causal)}")


# Continuation workloads: the last 2048-row chunk of the 16k sequence
# (chunked prefill against a 14k-token cache).
KV_WORKLOADS = {
    "chunk2048_t16384_d128": KVWorkload("chunk2048_t16384_d128", 1, 32, 8, 2048, 16384, 128),
}


@dataclass(frozen=True)
class RmsWorkload:
    """Fused RMSNorm over `rows` token rows of `n` features (bf16)."""
    name: str
    rows: int
    n: int
    eps: float = 1e-6
    seed: int = 0

    @property
    def bytes(self) -> float:
        """HBM bytes a pass must move: x read and y written once, w read once."""
        return 2.0 * (2 * self.rows * self.n + self.n)

    def describe(self) -> str:
        return f"rows={self.rows} n={self.n} bf16 eps={self.eps:g}"


# The 16k tokens of the long-context workload at its model width, Hq * D = 4096.
RMS_WORKLOADS = {
    "rmsnorm_16384x4096": RmsWorkload("rmsnorm_16384x4096", 16384, 4096),
}


@dataclass(frozen=True)
class PagedWorkload:
    """Decoding Tq new tokens for each of B sequences whose keys and values sit
    in a block-paged cache.  Cached lengths (the new tokens included) are drawn
    uniformly from [ctx_min, ctx_max]; the physical blocks of all sequences are
    a random permutation of the pool, `spare` blocks of which stay unused."""
    name: str
    B: int
    Hq: int
    Hkv: int
    Tq: int
    D: int
    block_size: int
    ctx_min: int
    ctx_max: int
    causal: bool = True
    spare: int = 64
    seed: int = 0

    @property
    def scale(self) -> float:
        return default_scale(self.D)

    @property
    def max_blocks(self) -> int:
        return -(-self.ctx_max // self.block_size)

    def describe(self) -> str:
        return (f"B={self.B} Hq={self.Hq} Hkv={self.Hkv} Tq={self.Tq} D={self.D} "
                f"block_size={self.block_size} context {self.ctx_min}..{self.ctx_max} bf16 "
                f"causal={int(self.causal)}")


# Decode steps of a serving batch at the long-context head shape: 64 sequences
# with 512 to 16384 cached tokens each, 16-token blocks.
PAGED_WORKLOADS = {
    "decode_b64_ctx16k_d128": PagedWorkload("decode_b64_ctx16k_d128", 64, 32, 8, 1, 128, 16,
                                            512, 16384),
}


def paged_bytes(context_lens, Hq, Hkv, Tq, D, block_size) -> float:
    """HBM bytes one decode call must move: every cached K and V row of every
    sequence once, q read, out and lse written, and the block-table entries
    in use read once (plus the length of each sequence)."""
    n = np.asarray(context_lens, dtype=np.int64)
    B = n.shape[0]
    kv = 2.0 * 2 * Hkv * D * float(n.sum())
    qo = 2.0 * 2 * B * Hq * Tq * D + 4.0 * B * Hq * Tq
    table = 4.0 * float((-(-n // block_size)).sum()) + 4.0 * B
    return kv + qo + table


def make_paged(B, Hq, Hkv, Tq, D, block_size, context_lens=None, ctx_range=None, spare=64,
               max_blocks=None, seed=0):
    """Inputs of one paged decode call, as CPU tensors:
    (q [B,Hq,Tq,D] bf16, k_cache, v_cache [num_blocks,Hkv,block_size,D] bf16,
    block_table [B,max_blocks] int32, context_lens [B] int32).

    Recipe, with default_rng(seed): the lengths (given, or drawn with
    integers(lo, hi + 1, size=B) from ctx_range = (lo, hi)); then a permutation
    of the num_blocks = used + spare physical blocks, whose first `used`
    entries go to the logical blocks of sequence 0, 1, ... in order; then
    standard_normal float32 draws of q, the K cache and the V cache, cast to
    bf16 (nearest even).  Table entries past a sequence's last block are -1."""
    rng = np.random.default_rng(seed)
    if context_lens is None:
        lo, hi = ctx_range
        context_lens = rng.integers(lo, hi + 1, size=B)
    lens = np.asarray(context_lens, dtype=np.int64)
    if lens.shape != (B,) or (lens < 0).any():
        raise ValueError("context_lens must be B non-negative lengths")
    nblk = -(-lens // block_size)
    if max_blocks is None:
        max_blocks = max(1, int(nblk.max()))
    if (nblk > max_blocks).any():
        raise ValueError("a sequence needs more blocks than max_blocks")
    used = int(nblk.sum())
    num_blocks = used + spare
    if num_blocks < 1:
        raise ValueError("the cache needs at least one block")
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((B, max_blocks), -1, dtype=np.int32)
    at = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[at:at + nblk[b]]
        at += int(nblk[b])
    q = rng.standard_normal((B, Hq, Tq, D), dtype=np.float32)
    kc = rng.standard_normal((num_blocks, Hkv, block_size, D), dtype=np.float32)
    vc = rng.standard_normal((num_blocks, Hkv, block_size, D), dtype=np.float32)
    bf = [torch.from_numpy(a).to(torch.bfloat16).contiguous() for a in (q, kc, vc)]
    return (bf[0], bf[1], bf[2], torch.from_numpy(table),
            torch.from_numpy(lens.astype(np.int32)))


def make_paged_workload(w: PagedWorkload):
    return make_paged(w.B, w.Hq, w.Hkv, w.Tq, w.D, w.block_size,
                      ctx_range=(w.ctx_min, w.ctx_max), spare=w.spare,
                      max_blocks=w.max_blocks, seed=w.seed)


def make_rmsnorm(rows, n, seed=0, scale=1.0):
    """x [rows, n] ~ scale * N(0,1) and w [n] ~ 1 + 0.5 * N(0,1), drawn in that
    order with default_rng(seed) in float32, then cast to bf16 (nearest even)."""
    rng = np.random.default_rng(seed)
    x = torch.from_numpy(rng.standard_normal((rows, n), dtype=np.float32) * np.float32(scale))
    w = torch.from_numpy(1.0 + 0.5 * rng.standard_normal(n, dtype=np.float32))
    return x.to(torch.bfloat16).contiguous(), w.to(torch.bfloat16).contiguous()


def default_scale(D: int) -> float:
    """The fp32 value of 1/sqrt(D), returned as a Python float."""
    return float(np.float32(1.0 / math.sqrt(D)))


def draw_fp32(B, Hq, Hkv, T, D, seed=0, outliers=""):
    """Q, K, V as float32 numpy arrays, drawn in the documented order."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, T, D), dtype=np.float32)
    if outliers == "elements":
        q[rng.random(q.shape) < OUTLIER_PROB] *= OUTLIER_FACTOR
        k[rng.random(k.shape) < OUTLIER_PROB] *= OUTLIER_FACTOR
    elif outliers == "rows":
        q[rng.random(q.shape[:3]) < OUTLIER_PROB] *= OUTLIER_FACTOR
        k[rng.random(k.shape[:3]) < OUTLIER_PROB] *= OUTLIER_FACTOR
    elif outliers:
        raise ValueError(f"unknown outlier mode {outliers!r}")
    return q, k, v


def make_qkv(B, Hq, Hkv, T, D, dtype="bf16", seed=0, outliers=""):
    """Q, K, V as contiguous CPU torch tensors of the requested dtype."""
    arrs = draw_fp32(B, Hq, Hkv, T, D, seed, outliers)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    return tuple(torch.from_numpy(a).to(tdt).contiguous() for a in arrs)


def make_qkv_on_device(B, Hq, Hkv, T, D, seed, device):
    """bf16 Q, K, V drawn on the GPU by torch's own seeded generator (Philox),
    for sizes whose host draw would take minutes: N(0,1) in the order Q, K, V.
    The draw is reproducible for a seed on one torch build; a test that uses
    it hands the oracle slices copied back from these very tensors."""
    return randn_on_device(((B, Hq, T, D), (B, Hkv, T, D), (B, Hkv, T, D)), seed, device)


def randn_on_device(shapes, seed, device):
    """bf16 N(0,1) tensors of the given shapes, drawn in order on the GPU by one
    torch generator seeded with `seed`."""
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return tuple(torch.randn(shape, generator=g, device=device, dtype=torch.bfloat16)
                 for shape in shapes)


def make_workload(w: Workload):
    return make_qkv(w.B, w.Hq, w.Hkv, w.T, w.D, w.dtype, w.seed, w.outliers)


def make_kv_workload(w: KVWorkload, full_q: bool = False):
    """(q, k, v) of a continuation workload: q holds the last Tq rows of the
    full query tensor (all Tk rows when full_q, for checks against a full
    forward)."""
    q, k, v = make_qkv(w.B, w.Hq, w.Hkv, w.Tk, w.D, w.dtype, w.seed)
    if not full_q:
        q = q[:, :, w.Tk - w.Tq:].contiguous()
    return q, k, v


def bits(t: torch.Tensor) -> np.ndarray:
    """The exact stored values of a CPU tensor, as the oracle takes them:
    float32 arrays for fp32, uint16 bit patterns for bf16."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.float32:
        return t.numpy()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    raise ValueError(f"unsupported dtype {t.dtype}")
