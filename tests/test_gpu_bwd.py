"""GPU parity of the attention backward (tessera_attn_bwd through the binding)
against the fp64 oracle.

The GPU forward supplies out and lse (as a training step would); the oracle
computes the exact gradients from q, k, v and dout alone.  Bar, per tensor X
of the reference (dq, dk, dv, Delta): max-abs error <= 2^-6 max|X| and
mean-abs error <= 2^-7 RMS(X).  The pages fix no precision for gradients; the
pipeline rounds P and dS to bf16 for the matrix cores, takes Delta from the
bf16 forward output, and rounds each result to bf16.  The oracle's arithmetic
with just those roundings added (a CPU emulation) lands at 0.2-0.5 % of
max|X| on N(0,1) inputs, and at 1.01 * 2^-7 max|dk| on the T=4096 workload
whose Q and K carry x8 outlier entries (dk sums many bf16-rounded dS terms
with large q entries); the GPU matches the emulation there.  The max-abs bar
is therefore two bf16 ulps of max|X|, the mean-abs bar one ulp of RMS(X)
(emulation and GPU at most 0.19 of it).
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


MAX_BAR = 2.0 ** -6    # of max|X|
MEAN_BAR = 2.0 ** -7   # of RMS(X)


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
    check_grads((dq, dk, dv, delta), r)


def check_grads(got_all, ref_all, what=""):
    """dq, dk, dv, Delta against the oracle's, each to the bar of its own
    largest and RMS value."""
    stats = []
    for name, got, ref in zip(("dq", "dk", "dv", "delta"), got_all, ref_all):
        g = got.float().cpu().numpy().astype(np.float64)
        assert np.isfinite(g).all(), name
        top, rms = float(np.abs(ref).max()), float(np.sqrt((ref ** 2).mean()))
        e = np.abs(g - ref)
        stats.append(f"{name} max {e.max():.2e} ({e.max() / max(top, 1e-30):.2%} of max) "
                     f"mean {e.mean():.2e} ({e.mean() / max(rms, 1e-30):.2%} of rms)")
        assert e.max() <= MAX_BAR * top and e.mean() <= MEAN_BAR * rms, (name, what, e.max(),
                                                                            e.mean(), top, rms)
    say(what, " | ".join(stats))


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
    (1, 16, 2, 200, 64, True),     # G = 8
    (2, 10, 2, 150, 128, False),   # G = 5, ragged, no mask
    (1, 32, 1, 96, 32, True),      # G = 32
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


def test_bwd_outlier_workload_slice():
    """The T=4096 workload with x8 outlier entries in Q and K (B=16 Hq=16 Hkv=4
    D=64), in the bench's launch: the whole batch on the GPU, the gradients of
    batch element 0, KV head 0 and its four query heads checked against the
    oracle (the bench's dout: torch.randn, seed 7)."""
    w = inputs.WORKLOADS["t4096_outliers"]
    q, k, v = inputs.make_workload(w)
    g = torch.Generator().manual_seed(7)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    say(f"case bwd workload {w.name}: {w.describe()}, slice b=0 KV head 0")
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    out, lse = binding.attn_fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    dq, dk, dv, delta = binding.attn_bwd(qd, kd, vd, out, lse, dod, causal=w.causal,
                                         scale=w.scale)
    torch.cuda.synchronize()
    G = w.Hq // w.Hkv
    r = oracle.attn_bwd(inputs.bits(q[:1, :G]), inputs.bits(k[:1, :1]), inputs.bits(v[:1, :1]),
                        inputs.bits(do[:1, :G]), w.causal, w.scale)
    stats = []
    for name, got, ref in zip(("dq", "dk", "dv", "delta"),
                              (dq[:1, :G], dk[:1, :1], dv[:1, :1], delta[:1, :G]), r):
        gv = got.float().cpu().numpy().astype(np.float64)
        top, rms = float(np.abs(ref).max()), float(np.sqrt((ref ** 2).mean()))
        e = np.abs(gv - ref)
        stats.append(f"{name} max {e.max() / (MAX_BAR * top):.3f} of bar, "
                     f"mean {e.mean() / (MEAN_BAR * rms):.3f} of bar")
        assert e.max() <= MAX_BAR * top and e.mean() <= MEAN_BAR * rms, (name, e.max(), e.mean())
    say(" | ".join(stats))


def test_bwd_long_context_sampled_rows():
    """The long-context workload (B=1 Hq=32 Hkv=8 T=16384 D=128) at full size,
    in the bench's launch: dq and Delta of 18 query rows (three heads, tile
    edges and the ends) and dk, dv of 6 key rows of KV head 3, each rebuilt by
    the oracle from the definitions.  The max-abs bar's scale, max|X|, is taken
    over the whole GPU tensor (the oracle cannot afford all rows); the
    mean-abs bar is a statistic of whole tensors and is left to the other
    tests (these rows lean on the shortest rows, whose errors are largest)."""
    w = inputs.WORKLOADS["t16384_d128"]
    q, k, v = inputs.make_workload(w)
    g = torch.Generator().manual_seed(7)
    do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
    say(f"case bwd workload {w.name}: {w.describe()}, sampled rows")
    dev = torch.device("cuda:0")
    qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
    out, lse = binding.attn_fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    dq, dk, dv, delta = binding.attn_bwd(qd, kd, vd, out, lse, dod, causal=w.causal,
                                         scale=w.scale)
    torch.cuda.synchronize()
    T = w.T
    qrows = np.array([h * T + i for h in (0, 13, 31) for i in (0, 1, 63, 64, T // 2 - 1, T - 1)],
                     np.int64)
    krows = np.array([3 * T + j for j in (0, 1, 127, 128, 8000, T - 1)], np.int64)
    rq, rd, rk, rv = oracle.attn_bwd_rows(inputs.bits(q), inputs.bits(k), inputs.bits(v),
                                          inputs.bits(do), w.causal, w.scale, qrows, krows)
    stats = []
    for name, full, rows, ref in (("dq", dq, qrows, rq), ("delta", delta, qrows, rd),
                                  ("dk", dk, krows, rk), ("dv", dv, krows, rv)):
        f = full.float().cpu().numpy().astype(np.float64)
        got = f.reshape(-1, w.D)[rows] if f.ndim == 4 else f.reshape(-1)[rows]
        top = float(np.abs(f).max())
        e = np.abs(got - ref)
        stats.append(f"{name} max {e.max() / (MAX_BAR * top):.3f} of bar")
        assert e.max() <= MAX_BAR * top, (name, e.max(), top)
    say(" | ".join(stats))


def test_bwd_offsets_past_int32():
    """Q, dO, O and dq of 8200 x 32 x 128 x 64 elements (more than 2^31): the
    last eight batch elements start past 2^31 elements.  Batch elements 0, 8192
    and the last are compared whole against the oracle."""
    B, Hq, Hkv, T, D = 8200, 32, 8, 128, 64
    assert B * Hq * T * D > 2 ** 31
    dev = torch.device("cuda:0")
    say(f"case bwd int32-overflowing offsets B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} causal")
    q, k, v = inputs.make_qkv_on_device(B, Hq, Hkv, T, D, seed=22, device=dev)
    (do,) = inputs.randn_on_device(((B, Hq, T, D),), seed=23, device=dev)
    scale = inputs.default_scale(D)
    out, lse = binding.attn_fwd(q, k, v, causal=True, scale=scale)
    dq, dk, dv, delta = binding.attn_bwd(q, k, v, out, lse, do, causal=True, scale=scale)
    torch.cuda.synchronize()
    for b in (0, 8192, B - 1):
        sl = [t[b:b + 1].cpu() for t in (q, k, v, do)]
        r = oracle.attn_bwd(*(inputs.bits(t) for t in sl), True, scale)
        check_grads(tuple(t[b:b + 1] for t in (dq, dk, dv, delta)), r, f"batch element {b}")
    del q, k, v, do, out, lse, dq, dk, dv, delta
    torch.cuda.empty_cache()
