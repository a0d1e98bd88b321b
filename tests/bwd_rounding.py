"""The attention backward in fp64 with the roundings of the bf16 GPU pipeline
added: the model from which the parity bar of the GPU backward is derived.

TEST-SIDE CODE.  It is independent of the HIP library (numpy only) and is
checked against the fp64 oracle with the roundings switched off.

The gradients are those of attention (page "Tessera: a from-scratch
distillation and serving stack in one repository", section "The kernel set
and its torch fallback", which lists the fused backward as missing):

    P  = softmax(scale Q K^T + mask)       dP = dO V^T
    Delta_i = sum_d dO_id O_id             dS = P (dP - Delta)
    dq = scale dS K     dk = scale dS^T Q     dv = P^T dO

summed over the query heads of a KV head for dk and dv.  The GPU pipeline
feeds its matrix cores bf16 operands, so on top of the exact arithmetic it
rounds (each to bf16, nearest even):
  * O, the forward output Delta is formed from (the forward returns bf16);
  * P, where it is the operand of dv = P^T dO;
  * dS, where it is the operand of dq and dk;
  * each of dq, dk, dv once at the end (after the multiplication by scale).
Everything else on the GPU is fp32, whose errors sit about 2^16 times below
these.  `backward(..., rounding=False)` is the exact backward; it must equal
the oracle to fp64 round-off.
"""
from __future__ import annotations

import math

import numpy as np
import torch

# The bar of the GPU backward, per tensor X (dq, dk, dv, Delta): max-abs error
# <= MAX_BAR * max|X| and mean-abs error <= MEAN_BAR * RMS(X).  Each is the
# smallest power of two at least HEADROOM times the worst ratio this model
# reaches over BAR_CASES and the T=4096 outlier slice (tests/test_bwd_bar.py
# recomputes both and checks that rule).  HEADROOM covers what the model
# leaves out: the GPU rounds its own fp32 values of P and dS, so a value next
# to a bf16 rounding boundary may round the other way, which moves the
# extreme of a tensor's errors by a fraction of one rounding.
HEADROOM = 1.5
MAX_BAR = 2.0 ** -6
MEAN_BAR = 2.0 ** -8

# (B, Hq, Hkv, T, D, causal): N(0,1) shapes with GQA groups 1, 2, 3, 4, 5, 6,
# 8 and 32, ragged T, causal and not; drawn by make_bwd with seed T + D.  The
# last four have more than 512 dk/dv workgroups (one per KV head and 128-key
# tile), two per CU on 256 CUs, so at D <= 64 they take the library's
# two-workgroups-per-CU dk/dv build; the smaller grids take its one-step-late
# build.
BAR_CASES = [
    (1, 4, 2, 64, 64, True),       # one tile
    (2, 8, 2, 128, 128, True),
    (1, 4, 1, 192, 32, True),      # MQA
    (2, 4, 4, 100, 64, True),      # MHA, ragged
    (1, 8, 2, 333, 128, True),     # ragged
    (1, 6, 2, 257, 64, False),     # G = 3, ragged, no mask
    (2, 8, 8, 64, 128, False),
    (1, 16, 4, 500, 64, True),
    (1, 12, 2, 130, 128, True),    # G = 6
    (1, 16, 2, 200, 64, True),     # G = 8
    (2, 10, 2, 150, 128, False),   # G = 5, ragged, no mask
    (1, 32, 1, 96, 32, True),      # G = 32
    (1, 80, 80, 900, 64, True),    # MHA, ragged: 640 dk/dv workgroups
    (5, 192, 64, 130, 64, False),  # G = 3, ragged, no mask: 640
    (3, 64, 32, 700, 32, True),    # ragged: 576
    (10, 16, 16, 400, 32, False),  # MHA, no mask: 640
]


def make_bwd(B, Hq, Hkv, T, D, seed):
    """bf16 q, k, v (the seeded N(0,1) recipe of the forward) and dO ~ N(0,1)
    drawn with default_rng(seed + 7), as CPU tensors."""
    from attention_flashattention_fwd_amd import inputs

    q, k, v = inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed)
    rng = np.random.default_rng(seed + 7)
    do = torch.from_numpy(rng.standard_normal((B, Hq, T, D), dtype=np.float32))
    return q, k, v, do.to(torch.bfloat16).contiguous()


def workload_dout(q: torch.Tensor) -> torch.Tensor:
    """The output gradient of the full-size backward workloads: torch.randn
    shaped like q from a CPU generator seeded with 7, cast to bf16."""
    g = torch.Generator().manual_seed(7)
    return torch.randn(q.shape, generator=g).to(torch.bfloat16)


def smallest_power_of_two_at_least(x: float) -> float:
    return 2.0 ** math.ceil(math.log2(x))


def bf16_round(x: np.ndarray) -> np.ndarray:
    """x rounded to bfloat16 (to fp32, then to 8 significant bits, nearest
    even), returned as float64.  Inputs are finite."""
    u = np.ascontiguousarray(x, dtype=np.float64).astype(np.float32).view(np.uint32)
    u = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) & np.uint32(0xFFFF0000)
    return u.view(np.float32).astype(np.float64)


def bf16_values(bits: np.ndarray) -> np.ndarray:
    """float64 values of an array of bf16 bit patterns (uint16)."""
    return (bits.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def backward(q, k, v, do, causal: bool, scale: float, rounding: bool = True):
    """Gradients (dq, dk, dv, Delta) for float64 q, do [B,Hq,T,D] and k, v
    [B,Hkv,T,D]; with `rounding`, the bf16 roundings listed above are applied
    where the GPU pipeline makes them."""
    B, Hq, T, D = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    r = bf16_round if rounding else (lambda a: a)
    dq = np.empty_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    delta = np.empty((B, Hq, T))
    hidden = np.triu(np.ones((T, T), dtype=bool), 1) if causal else None
    for b in range(B):
        for h in range(Hq):
            g = h // G
            K, V, Q, dO = k[b, g], v[b, g], q[b, h], do[b, h]
            S = scale * (Q @ K.T)
            if causal:
                S[hidden] = -np.inf
            E = np.exp(S - S.max(axis=1, keepdims=True))
            P = E / E.sum(axis=1, keepdims=True)
            O = r(P @ V)
            dl = np.sum(dO * O, axis=1)
            dS = r(P * (dO @ V.T - dl[:, None]))
            dq[b, h] = scale * (dS @ K)
            dk[b, g] += scale * (dS.T @ Q)
            dv[b, g] += r(P).T @ dO
            delta[b, h] = dl
    if rounding:
        dq, dk, dv = r(dq), r(dk), r(dv)
    return dq, dk, dv, delta


def error_ratios(got, ref):
    """(max-abs error / max|ref|, mean-abs error / RMS(ref)) of one tensor."""
    e = np.abs(got - ref)
    return float(e.max() / np.abs(ref).max()), float(e.mean() / np.sqrt(np.mean(ref * ref)))
