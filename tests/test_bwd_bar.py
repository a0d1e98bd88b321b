"""Derivation of the parity bar of the GPU attention backward (CPU only).

The bar comes from tests/bwd_rounding.py: the exact backward in fp64 with the
bf16 roundings the GPU pipeline makes (O for Delta, P for dv, dS for dq and
dk, each result once).  These tests
  * pin that model to the oracle (with the roundings off it is the oracle, to
    fp64 round-off) and to the bf16 rounding rule itself;
  * recompute its error on the N(0,1) cases of the GPU tests and on the slice
    of the T=4096 outlier workload that the GPU test checks, and check that
    MAX_BAR and MEAN_BAR are the smallest powers of two at least HEADROOM
    times the worst ratios (so the bar follows from the model, and is not
    looser than that rule).
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from attention_flashattention_fwd_amd import inputs
from tests import bwd_rounding as br


def _bits(*ts):
    return [inputs.bits(t) for t in ts]


def test_bf16_round_is_nearest_even():
    # torch's float32 -> bfloat16 cast rounds to nearest even: an independent check
    rng = np.random.default_rng(3)
    x = np.concatenate([rng.standard_normal(100000) * 10.0 ** rng.integers(-8, 8, 100000),
                        [1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -(1.0 + 2.0 ** -8), 0.0]])
    want = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).float().numpy()
    assert np.array_equal(br.bf16_round(x), want.astype(np.float64))
    assert br.bf16_round(np.array([1.0 + 2.0 ** -8]))[0] == 1.0             # tie to even
    assert br.bf16_round(np.array([1.0 + 3 * 2.0 ** -8]))[0] == 1.0 + 2.0 ** -6


@pytest.mark.parametrize("case", br.BAR_CASES[:6])
def test_model_without_rounding_is_the_oracle(case):
    B, Hq, Hkv, T, D, causal = case
    q, k, v, do = br.make_bwd(B, Hq, Hkv, T, D, seed=T + D)
    bits = _bits(q, k, v, do)
    scale = inputs.default_scale(D)
    ref = oracle.attn_bwd(*bits, causal, scale)
    got = br.backward(*(br.bf16_values(b) for b in bits), causal, scale, rounding=False)
    for name, a, r in zip(("dq", "dk", "dv", "delta"), got, ref):
        assert np.abs(a - r).max() <= 1e-12 * max(np.abs(r).max(), 1.0), name


def test_rounding_moves_the_result_by_about_one_bf16_rounding():
    # the model with roundings differs from the exact backward, by far less
    # than the bar (a model that rounded nothing would make the bar unfounded)
    B, Hq, Hkv, T, D, causal = br.BAR_CASES[1]
    q, k, v, do = br.make_bwd(B, Hq, Hkv, T, D, seed=T + D)
    vals = [br.bf16_values(b) for b in _bits(q, k, v, do)]
    scale = inputs.default_scale(D)
    ex = br.backward(*vals, causal, scale, rounding=False)
    em = br.backward(*vals, causal, scale, rounding=True)
    for a, r in zip(em, ex):
        mx, mean = br.error_ratios(a, r)
        assert 2.0 ** -12 < mx < br.MAX_BAR and 2.0 ** -14 < mean < br.MEAN_BAR


def emulated_worst():
    """Worst (max, mean) error ratios of the rounding model against the
    oracle over the N(0,1) cases and the T=4096 outlier slice, per case."""
    rows = []
    for case in br.BAR_CASES:
        B, Hq, Hkv, T, D, causal = case
        q, k, v, do = br.make_bwd(B, Hq, Hkv, T, D, seed=T + D)
        bits = _bits(q, k, v, do)
        scale = inputs.default_scale(D)
        ref = oracle.attn_bwd(*bits, causal, scale)
        em = br.backward(*(br.bf16_values(b) for b in bits), causal, scale)
        rows.append((str(case), [br.error_ratios(a, r) for a, r in zip(em, ref)]))
    w = inputs.WORKLOADS["t4096_outliers"]
    q, k, v = inputs.make_workload(w)
    do = br.workload_dout(q)
    G = w.Hq // w.Hkv
    bits = _bits(q[:1, :G], k[:1, :1], v[:1, :1], do[:1, :G])
    ref = oracle.attn_bwd(*bits, w.causal, w.scale)
    em = br.backward(*(br.bf16_values(b) for b in bits), w.causal, w.scale)
    rows.append(("t4096_outliers b=0 KV head 0", [br.error_ratios(a, r) for a, r in zip(em, ref)]))
    return rows


def test_bar_follows_from_the_rounding_model():
    rows = emulated_worst()
    for name, ratios in rows:
        print(name, " | ".join(f"{n} max {a / 2 ** -7:.3f} mean {m / 2 ** -7:.3f} (x 2^-7)"
                               for n, (a, m) in zip(("dq", "dk", "dv", "delta"), ratios)))
    worst_max = max(a for _, r in rows for a, _ in r)
    worst_mean = max(m for _, r in rows for _, m in r)
    print(f"worst: max {worst_max / 2 ** -7:.3f}, mean {worst_mean / 2 ** -7:.3f} (x 2^-7)")
    assert br.MAX_BAR == br.smallest_power_of_two_at_least(br.HEADROOM * worst_max)
    assert br.MEAN_BAR == br.smallest_power_of_two_at_least(br.HEADROOM * worst_mean)
    # the outlier slice is where the max-abs ratio peaks (dk: large q entries
    # weight many rounded dS terms)
    assert max(a for a, _ in rows[-1][1]) == worst_max


def test_cases_cover_both_dkdv_builds_at_small_head_sizes():
    # The library takes its one-step-late dk/dv build at D <= 64 on grids of at
    # most two dk/dv workgroups (one per KV head and 128-key tile) per compute
    # unit, its two-workgroups-per-CU build above: on the 256 CUs of an MI355X
    # the boundary is 512.  The GPU cases must reach both builds at D = 64 and
    # D = 32, causal or not among them.
    def grid(case):
        B, Hq, Hkv, T, D, causal = case
        return B * Hkv * -(-T // 128)

    for D in (32, 64):
        small = [c for c in br.BAR_CASES if c[4] == D and grid(c) <= 2 * 256]
        large = [c for c in br.BAR_CASES if c[4] == D and grid(c) > 2 * 256]
        assert small and large, D
        assert {c[5] for c in large} == {True, False}, D
