"""Pins of the fp64 attention-backward oracle to facts other than itself.

  * torch autograd in float64 on the CPU through an explicit masked softmax
    (an independent library computation), K/V heads repeated for GQA;
  * central finite differences of L = sum(O * dO) through the forward oracle
    (itself pinned), on fp32 inputs stepped by an exactly representable h;
  * closed forms: the dv rows of a KV head add up to the dO rows of its query
    heads (each softmax row sums to one); the dk rows add up to zero (softmax
    is unchanged by adding one vector to every key); Delta equals the row sums
    of dO * O with O from the forward oracle;
  * GQA equals repeated-head MHA with dk, dv summed over the repeats;
  * the selected-rows entry (dq, Delta of chosen query rows, dk, dv of chosen
    key rows, each rebuilt from the definitions) equals the rows of the full
    call.
"""
from __future__ import annotations

import math

import numpy as np
import torch

from tests.oracle_pins import as_dtype, rand_inputs, values


def rand_bwd(B, Hq, Hkv, T, D, seed):
    q, k, v = rand_inputs(B, Hq, Hkv, T, D, "bf16", seed)
    rng = np.random.default_rng(seed + 1000)
    do = as_dtype(rng.standard_normal((B, Hq, T, D)).astype(np.float32), "bf16")
    return q, k, v, do


def torch_grads(q, k, v, do, causal, scale):
    G = q.shape[1] // k.shape[1]
    qt, kt, vt, dot = (torch.from_numpy(values(a)).requires_grad_(True) for a in (q, k, v, do))
    kr, vr = kt.repeat_interleave(G, dim=1), vt.repeat_interleave(G, dim=1)
    s = (qt @ kr.transpose(-1, -2)) * scale
    if causal:
        T = q.shape[2]
        s = s.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
    o = torch.softmax(s, dim=-1) @ vr
    (o * dot.detach()).sum().backward()
    return qt.grad.numpy(), kt.grad.numpy(), vt.grad.numpy(), o.detach().numpy()


def pin_bwd_torch_autograd(lib):
    for n, (B, Hq, Hkv, T, D, causal) in enumerate([(2, 4, 2, 13, 8, True), (1, 6, 2, 21, 16, False),
                                                    (1, 2, 2, 40, 32, True)]):
        q, k, v, do = rand_bwd(B, Hq, Hkv, T, D, seed=800 + n)
        scale = float(np.float32(1.0 / math.sqrt(D)))
        dq, dk, dv, _ = lib.attn_bwd(q, k, v, do, causal, scale)
        tq, tk, tv, _ = torch_grads(q, k, v, do, causal, scale)
        for name, a, b in (("dq", dq, tq), ("dk", dk, tk), ("dv", dv, tv)):
            assert np.abs(a - b).max() <= 1e-11, (name, B, Hq, Hkv, T, D, causal)


def pin_bwd_finite_differences(lib):
    """d/dx of L = sum(O * dO) by central differences with h = 2^-10 on fp32
    inputs (x +- h is exact for these magnitudes), through the forward oracle."""
    B, Hq, Hkv, T, D, causal, scale = 1, 4, 2, 6, 4, True, 0.7
    q, k, v, do = rand_bwd(B, Hq, Hkv, T, D, seed=9)
    dq, dk, dv, _ = lib.attn_bwd(q, k, v, do, causal, scale)
    f32 = [values(a).astype(np.float32) for a in (q, k, v)]
    dov = values(do)
    h = 2.0 ** -10
    rng = np.random.default_rng(3)

    def loss(arrs):
        O, _ = lib.attn_fwd(*arrs, causal, scale)
        return float((O * dov).sum())

    for which, grad in ((0, dq), (1, dk), (2, dv)):
        for _ in range(6):
            idx = tuple(int(rng.integers(0, s)) for s in f32[which].shape)
            plus = [a.copy() for a in f32]
            minus = [a.copy() for a in f32]
            plus[which][idx] += np.float32(h)
            minus[which][idx] -= np.float32(h)
            assert plus[which][idx] - f32[which][idx] == np.float32(h)
            fd = (loss(plus) - loss(minus)) / (2 * h)
            assert abs(fd - grad[idx]) <= 1e-5 * max(1.0, abs(grad[idx])), (which, idx, fd,
                                                                               grad[idx])


def pin_bwd_closed_forms(lib):
    B, Hq, Hkv, T, D = 2, 6, 3, 17, 8
    q, k, v, do = rand_bwd(B, Hq, Hkv, T, D, seed=11)
    G = Hq // Hkv
    for causal in (True, False):
        dq, dk, dv, delta = lib.attn_bwd(q, k, v, do, causal, 0.4)
        dov = values(do)
        want_dv = dov.reshape(B, Hkv, G, T, D).sum(axis=(2, 3))
        assert np.abs(dv.sum(axis=2) - want_dv).max() <= 1e-12
        assert np.abs(dk.sum(axis=2)).max() <= 1e-12
        O, _ = lib.attn_fwd(q, k, v, causal, 0.4)
        assert np.abs(delta - (dov * O).sum(axis=-1)).max() <= 1e-12


def pin_bwd_gqa_equals_repeated_mha(lib):
    B, Hq, Hkv, T, D = 1, 4, 2, 11, 8
    q, k, v, do = rand_bwd(B, Hq, Hkv, T, D, seed=12)
    G = Hq // Hkv
    kr, vr = (np.ascontiguousarray(np.repeat(a, G, axis=1)) for a in (k, v))
    for causal in (True, False):
        dq, dk, dv, delta = lib.attn_bwd(q, k, v, do, causal, 0.3)
        mq, mk, mv, md = lib.attn_bwd(q, kr, vr, do, causal, 0.3)
        assert np.abs(dq - mq).max() <= 1e-13 and np.abs(delta - md).max() <= 1e-13
        assert np.abs(dk - mk.reshape(B, Hkv, G, T, D).sum(axis=2)).max() <= 1e-13
        assert np.abs(dv - mv.reshape(B, Hkv, G, T, D).sum(axis=2)).max() <= 1e-13


def pin_bwd_rows_entry(lib):
    for causal in (True, False):
        B, Hq, Hkv, T, D = 2, 6, 2, 37, 16
        q, k, v, do = rand_bwd(B, Hq, Hkv, T, D, seed=61 + int(causal))
        dq, dk, dv, delta = lib.attn_bwd(q, k, v, do, causal, 0.3)
        qrows = np.array([0, 1, T - 1, T, 2 * T + 17, B * Hq * T - 1], np.int64)
        krows = np.array([0, 5, T - 1, T + 3, 3 * T + 36, B * Hkv * T - 1], np.int64)
        rq, rd, rk, rv = lib.attn_bwd_rows(q, k, v, do, causal, 0.3, qrows, krows)
        assert np.abs(rq - dq.reshape(-1, D)[qrows]).max() <= 1e-12, causal
        assert np.abs(rd - delta.reshape(-1)[qrows]).max() <= 1e-12, causal
        assert np.abs(rk - dk.reshape(-1, D)[krows]).max() <= 1e-12, causal
        assert np.abs(rv - dv.reshape(-1, D)[krows]).max() <= 1e-12, causal


ALL_BWD_PINS = [pin_bwd_rows_entry, pin_bwd_torch_autograd, pin_bwd_finite_differences,
                pin_bwd_closed_forms, pin_bwd_gqa_equals_repeated_mha]
