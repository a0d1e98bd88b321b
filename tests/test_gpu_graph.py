"""Entry points captured into a HIP graph (torch.cuda.CUDAGraph) and replayed.

The library enqueues only kernel launches on the caller's stream (no memset,
copy or allocation), so its calls can be captured.  A bf16 forward that runs
persistently when called directly (work-queue counters) runs as a plain grid
under capture, with the same bits.  Each graph is replayed several times with
eager calls of the library and plain torch work in between, and every replay
must equal the eager result bit for bit.  (The eager results themselves are
checked against the oracle by the other GPU tests.)
"""
from __future__ import annotations

import pytest
import torch

from attention_flashattention_fwd_amd import binding, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")
REPLAYS = 3


def say(*msg):
    print(*msg, flush=True)


def capture(fn):
    """Warms fn up on a side stream, then captures one call of it."""
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def replay_and_check(g, outs, want, between):
    for r in range(REPLAYS):
        for o in outs:
            o.fill_(-7)   # stale values must not survive a replay
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for i, (o, w) in enumerate(zip(outs, want)):
            assert torch.equal(o, w), f"replay {r}: output {i} differs from the eager call"
        between()
        torch.cuda.synchronize()


def test_forward_persistent_shape_in_a_graph():
    # 1056 work items: persistent when called directly, a plain grid under capture
    B, Hq, Hkv, T, D = 8, 16, 4, 2112, 128
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=3))
    assert binding.tile_config(B, Hq, Hkv, T, T, D, 1).persistent == 1
    want = binding.attn_fwd(q, k, v, causal=True)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=DEV)
    say(f"case graph forward B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    g = capture(lambda: binding.attn_fwd_into(q, k, v, out, lse, True, None))
    other_o, other_l = torch.empty_like(q), torch.empty_like(lse)

    def between():
        binding.attn_fwd_into(q, k, v, other_o, other_l, True, None)   # eager, persistent
        (other_o.float() * 2).sum()                                      # unrelated torch work
    replay_and_check(g, [out, lse], list(want), between)
    assert torch.equal(other_o, want[0]) and torch.equal(other_l, want[1])


def test_backward_in_a_graph():
    B, Hq, Hkv, T, D = 1, 8, 2, 1000, 64
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=4))
    do = torch.randn((B, Hq, T, D), generator=torch.Generator().manual_seed(4)).to(
        torch.bfloat16).to(DEV)
    out, lse = binding.attn_fwd(q, k, v, causal=True)
    want = binding.attn_bwd(q, k, v, out, lse, do, causal=True)
    bufs = [torch.empty_like(q), torch.empty_like(k), torch.empty_like(v),
            torch.empty((B, Hq, T), dtype=torch.float32, device=DEV)]
    scale = inputs.default_scale(D)

    def call():
        st = binding.raw_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                             do.data_ptr(), lse.data_ptr(), *(b.data_ptr() for b in bufs),
                             B, Hq, Hkv, T, D, 1, scale,
                             torch.cuda.current_stream().cuda_stream)
        assert st == binding.OK, st
    say(f"case graph backward B={B} Hq={Hq} Hkv={Hkv} T={T} D={D}")
    g = capture(call)
    replay_and_check(g, bufs, list(want),
                     lambda: binding.attn_bwd(q, k, v, out, lse, do, causal=True))


def test_paged_decode_without_workspace_in_a_graph():
    lens = [1, 15, 700, 3000, 0, 129]
    q, kc, vc, table, cl = (t.to(DEV) for t in inputs.make_paged(
        len(lens), 16, 4, 2, 128, 16, context_lens=lens, spare=3, seed=5))
    want_o = torch.empty_like(q)
    want_l = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
    binding.paged_decode_noalloc_into(q, kc, vc, table, cl, want_o, want_l)   # first call: setup
    torch.cuda.synchronize()
    out, lse = torch.empty_like(want_o), torch.empty_like(want_l)
    say(f"case graph paged decode (no workspace) lens={lens}")
    g = capture(lambda: binding.paged_decode_noalloc_into(q, kc, vc, table, cl, out, lse))
    other_o, other_l = torch.empty_like(want_o), torch.empty_like(want_l)

    def between():
        # an eager call in between reuses the same library scratch
        binding.paged_decode_noalloc_into(q, kc, vc, table, cl, other_o, other_l)
    replay_and_check(g, [out, lse], [want_o, want_l], between)
    assert torch.equal(other_o, want_o) and torch.equal(other_l, want_l)


def test_rmsnorm_in_a_graph():
    x, w = (t.to(DEV) for t in inputs.make_rmsnorm(300, 4096, seed=6))
    want = binding.rmsnorm_fwd(x, w)
    y = torch.empty_like(x)
    say("case graph rmsnorm 300 x 4096")
    g = capture(lambda: binding.rmsnorm_fwd_into(x, w, y))
    replay_and_check(g, [y], [want], lambda: binding.rmsnorm_fwd(x, w))
