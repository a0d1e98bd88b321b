"""GPU parity of the attention backward (tessera_attn_bwd through the binding)
against the fp64 oracle.

The GPU forward supplies out and lse (as a training step would); the oracle
computes the exact gradients from q, k, v and dout alone.  Bar, per tensor X
of the reference (dq, dk, dv, Delta): max-abs error <= 2^-7 max|X| and
mean-abs error <= 2^-7 RMS(X), one bf16 ulp of the tensor's own scale.  The
pipeline rounds P and dS to bf16 for the matrix cores, takes Delta from the
bf16 forward output, and rounds each result to bf16; the oracle's arithmetic
with just those roundings added (a CPU check) already lands at 0.2-0.5 % of
max|X| and 0.2-0.3 % of RMS(X), the size of what the GPU shows.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from attention_flashattention_fwd_amd import binding, inputs
from tests.test_gpu_parity import say

pytestmark = pytest.mark.gpu


def make_bwd(B, Hq, Hkv, T, D, seed):
    q, k, v = inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed)
    rng = np.random.default_rng(seed + 7)
    do = torch.from_numpy(rng.standard_normal((B, Hq, T, D), dtype=np.float32))
    return q, k, v, do.to(torch.bfloat16).contiguous()


def run_case(B, Hq, Hkv, T, D, causal, seed, scale=None):
    scale = inputs.default_scale(D) if scale is None else scale
    q, k, v, do = make_bwd(B, Hq, Hkv, T, D, seed)
    say(f"case bwd B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} causal={causal} scale={scale}")
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    out, lse = binding.attn_fwd(qd, kd, vd, causal=causal, scale=scale)
    dq, dk, dv, delta = binding.attn_bwd(qd, kd, vd, out, lse, dod, causal=causal, scale=scale)
    torch.cuda.synchronize()
    r = oracle.attn_bwd(inputs.bits(q), inputs.bits(k), inputs.bits(v), inputs.bits(do), causal,
                        scale)
    stats = []
    for name, got, ref in zip(("dq", "dk", "dv", "delta"), (dq, dk, dv, delta), r):
        g = got.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all(), name
        top, rms = float(np.abs(ref).max()), float(np.sqrt((ref ** 2).mean()))
        e = np.abs(g - ref)
        stats.append(f"{name} max {e.max():.2e} ({e.max() / max(top, 1e-30):.2%} of max) "
                     f"mean {e.mean():.2e} ({e.mean() / max(rms, 1e-30):.2%} of rms)")
        assert e.max() <= 2.0 ** -7 * top and e.mean() <= 2.0 ** -7 * rms, (name, e.max(),
                                                                              e.mean(), top, rms)
    say(" | ".join(stats))


CASES = [
    (1, 4, 2, 64, 64, True),       # one tile
    (2, 8, 2, 128, 128, True),
    (1, 4, 1, 192, 32, True),      # MQA
    (2, 4, 4, 100, 64, True),      # MHA, ragged
    (1, 8, 2, 333, 128, True),     # ragged
    (1, 6, 2, 257, 64, False),     # G = 3, ragged, no mask
    (2, 8, 8, 64, 128, False),
    (1, 16, 4, 500, 64, True),
    (1, 12, 2, 130, 128, True),    # G = 6
]


@pytest.mark.parametrize("B,Hq,Hkv,T,D,causal", CASES)
def test_bwd_shapes(B, Hq, Hkv, T, D, causal):
    run_case(B, Hq, Hkv, T, D, causal, seed=T + D)


@pytest.mark.parametrize("scale", [-0.2, 0.0, 0.5])
def test_bwd_scale_values(scale):
    run_case(1, 8, 2, 150, 64, True, seed=4, scale=scale)


def test_bwd_repeatable():
    q, k, v, do = (t.cuda() for t in make_bwd(1, 8, 2, 300, 128, seed=2))
    out, lse = binding.attn_fwd(q, k, v)
    a = binding.attn_bwd(q, k, v, out, lse, do)
    b = binding.attn_bwd(q, k, v, out, lse, do)
    torch.cuda.synchronize()
    assert all(torch.equal(x, y) for x, y in zip(a, b))
