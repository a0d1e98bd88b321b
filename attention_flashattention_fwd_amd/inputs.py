"""Seeded synthetic inputs for the attention forward workloads.

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
