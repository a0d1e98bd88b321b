"""GPU parity of tessera_attn_fwd_kv (Tq query rows against Tk cached key rows)
against the fp64 oracle, through the C ABI.  Same bar as the full forward:
bf16 max-abs <= 2e-2 and mean-abs <= 2e-3 for O and lse."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from attention_flashattention_fwd_amd import binding, inputs
from tests.test_gpu_parity import check_close, say

pytestmark = pytest.mark.gpu


def make_kv(B, Hq, Hkv, Tq, Tk, D, seed):
    """Seeded N(0,1) draws rounded to bf16: q [B,Hq,Tq,D], k and v [B,Hkv,Tk,D]."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Tq, D), dtype=np.float32)
    k = rng.standard_normal((B, Hkv, Tk, D), dtype=np.float32)
    v = rng.standard_normal((B, Hkv, Tk, D), dtype=np.float32)
    return tuple(torch.from_numpy(a).to(torch.bfloat16).contiguous() for a in (q, k, v))


def run_kv(q, k, v, causal, scale):
    dev = torch.device("cuda:0")
    out, lse = binding.attn_fwd_kv(q.to(dev), k.to(dev), v.to(dev), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


CASES = [
    (1, 8, 2, 1, 333, 128, True),      # decode one token, ragged Tk
    (3, 8, 2, 5, 64, 64, True),        # a few tokens, one key tile
    (2, 8, 2, 17, 256, 64, True),
    (1, 4, 1, 64, 640, 32, True),      # MQA
    (2, 6, 2, 100, 1000, 128, True),   # G=3, ragged
    (1, 12, 2, 250, 1031, 64, True),   # G=6
    (2, 8, 2, 50, 200, 64, False),
    (1, 4, 4, 300, 129, 64, False),    # non-causal, more query rows than key rows
    (1, 8, 8, 96, 96, 128, True),      # Tq = Tk
]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,Tk,D,causal", CASES)
def test_kv_shapes(B, Hq, Hkv, Tq, Tk, D, causal):
    q, k, v = make_kv(B, Hq, Hkv, Tq, Tk, D, seed=Tq * 7 + Tk)
    scale = inputs.default_scale(D)
    say(f"case kv B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D} causal={causal}")
    o, l = run_kv(q, k, v, causal, scale)
    O_ref, l_ref = oracle.attn_fwd_kv(inputs.bits(q), inputs.bits(k), inputs.bits(v), causal,
                                      scale)
    check_close(o, l, O_ref, l_ref, "bf16")


def test_kv_two_workgroups_per_cu():
    """D = 64 with Tk a multiple of 64 on a 2048-workgroup grid: the paired build."""
    B, Hq, Hkv, Tq, Tk, D = 128, 64, 16, 64, 128, 64
    q, k, v = make_kv(B, Hq, Hkv, Tq, Tk, D, seed=3)
    scale = inputs.default_scale(D)
    say(f"case kv paired B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} Tk={Tk} D={D}")
    o, l = run_kv(q, k, v, True, scale)
    O_ref, l_ref = oracle.attn_fwd_kv(inputs.bits(q), inputs.bits(k), inputs.bits(v), True, scale)
    check_close(o, l, O_ref, l_ref, "bf16")


def test_kv_equals_full_forward_when_tq_equals_tk():
    """tessera_attn_fwd(T) is tessera_attn_fwd_kv(Tq = Tk = T): same bits."""
    q, k, v = (t.cuda() for t in inputs.make_qkv(2, 8, 2, 200, 64, "bf16", seed=9))
    for causal in (True, False):
        o1, l1 = binding.attn_fwd(q, k, v, causal=causal)
        o2, l2 = binding.attn_fwd_kv(q, k, v, causal=causal)
        torch.cuda.synchronize()
        assert torch.equal(o1, o2) and torch.equal(l1, l2)


def test_kv_suffix_matches_full_forward():
    """The serving invariant on the GPU path: new rows against the cache equal
    the same rows of a full forward, each within the bar of the oracle."""
    B, Hq, Hkv, T, D = 1, 8, 2, 700, 128
    q, k, v = inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=12)
    scale = inputs.default_scale(D)
    O_ref, l_ref = oracle.attn_fwd(inputs.bits(q), inputs.bits(k), inputs.bits(v), True, scale)
    for Tq in (1, 7, 64, 130):
        qs = q[:, :, T - Tq:].contiguous()
        say(f"case kv suffix T={T} Tq={Tq}")
        o, l = run_kv(qs, k, v, True, scale)
        check_close(o, l, O_ref[:, :, T - Tq:], l_ref[:, :, T - Tq:], "bf16")


def test_kv_argument_checks():
    q, k, v = (t.cuda() for t in make_kv(1, 4, 2, 10, 8, 64, seed=1))
    with pytest.raises(RuntimeError, match="bad shape"):
        binding.attn_fwd_kv(q, k, v, causal=True)     # causal with Tq > Tk
    out, lse = binding.attn_fwd_kv(q, k, v, causal=False)
    torch.cuda.synchronize()
    assert out.shape == q.shape and lse.shape == (1, 4, 10)
    with pytest.raises(ValueError):
        binding.attn_fwd_kv(q.float(), k.float(), v.float())


@pytest.mark.parametrize("name", sorted(inputs.KV_WORKLOADS))
def test_kv_full_size_workload(name):
    """The benchmarked continuation workload at its real size: every element of
    out and lse against the oracle's continuation (the rows of the full
    forward they belong to)."""
    w = inputs.KV_WORKLOADS[name]
    say(f"workload {name}: {w.describe()}, every element")
    q, k, v = inputs.make_kv_workload(w)
    dev = torch.device("cuda:0")
    out, lse = binding.attn_fwd_kv(q.to(dev), k.to(dev), v.to(dev), causal=w.causal,
                                   scale=w.scale)
    torch.cuda.synchronize()
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    O_ref, l_ref = oracle.attn_fwd_kv(inputs.bits(q), inputs.bits(k), inputs.bits(v), w.causal,
                                      w.scale)
    check_close(out.float().cpu().numpy().astype(np.float64),
                lse.cpu().numpy().astype(np.float64), O_ref, l_ref, w.dtype, name)
