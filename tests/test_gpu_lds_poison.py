"""The LDS-poisoned debug build (libtessera_attn_poison.so) against the
production library, through the C ABI.

In the debug build every kernel fills its LDS with a NaN pattern before its
first LDS access, and every global->LDS load writes the pattern over its
destination before it is issued.  A read that the kernel's hand-placed waits
and barriers let through too early (before its data landed, or after the
buffer's refill was issued) then reads NaN, which the products carry into the
outputs.  A correct kernel never reads the pattern, so each output must be
finite and equal to the production build's bit for bit (the arithmetic is the
same; the production outputs themselves are checked against the oracle by the
other GPU tests).  The cases run every forward tile configuration the sizes
allow (plain and persistent launches, one and two workgroups per CU, 32 and
64 query rows per wave, 1, 2 and 4 heads per workgroup), ragged and whole
tiles, the continuation, fp32, the backward and the paged decode.
"""
from __future__ import annotations

import itertools

import numpy as np
import pytest
import torch

from attention_flashattention_fwd_amd import binding, inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def say(*msg):
    print(*msg, flush=True)


def both(run):
    """run() under the production and the poisoned library; returns both
    results as lists of CPU tensors."""
    prod = [t.cpu() for t in run()]
    with binding.use_library(binding.POISON_LIBRARY):
        pois = [t.cpu() for t in run()]
    torch.cuda.synchronize()
    return prod, pois


def same(prod, pois, what, finite=True):
    for i, (a, b) in enumerate(zip(prod, pois)):
        if finite:
            assert torch.isfinite(b).all(), f"{what}: output {i} of the poisoned build is not finite"
        # bitwise, NaN and -inf included
        assert torch.equal(a.view(torch.uint8), b.view(torch.uint8)), \
            f"{what}: output {i} differs from the production build"


def test_poison_library_is_the_debug_build():
    with binding.use_library(binding.POISON_LIBRARY) as L:
        assert L._name == str(binding.POISON_LIBRARY)
        assert binding.version() == 10200
    assert binding.lib()._name == str(binding.LIBRARY)


CONFIGS = [binding.TileConfig(hg, rows, wpc, pers)
           for hg, rows, wpc, pers in itertools.product((1, 2, 4), (32, 64), (1, 2), (0, 1))]


# 1056 work items at four heads per workgroup (more at fewer), several per
# workgroup of a persistent launch, so its per-item refills of the ring run.
@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("T", [2100, 2112])
@pytest.mark.parametrize("causal", [True, False])
def test_poison_forward_every_config(D, T, causal):
    B, Hq, Hkv = 8, 16, 4
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=D + T))
    scale = inputs.default_scale(D)
    ran = []
    for cfg in CONFIGS:
        def run():
            o = torch.empty_like(q)
            l = torch.empty((B, Hq, T), device=DEV, dtype=torch.float32)
            st = binding.raw_fwd_with_config(q.data_ptr(), k.data_ptr(), v.data_ptr(),
                                             o.data_ptr(), l.data_ptr(), B, Hq, Hkv, T, T, D,
                                             int(causal), scale, cfg,
                                             torch.cuda.current_stream().cuda_stream)
            return (o, l) if st == binding.OK else ()
        prod, pois = both(run)
        assert len(prod) == len(pois)
        if not prod:
            continue
        ran.append(cfg.as_tuple())
        same(prod, pois, f"fwd D={D} T={T} causal={causal} {cfg}")
    say(f"case poison fwd D={D} T={T} causal={causal}: {len(ran)} configurations {ran}")
    # every build the sizes allow ran: plain and persistent, 1/2/4 heads per
    # workgroup, 64 rows per wave at D <= 64, two workgroups per CU at D <= 64
    # with whole key tiles
    assert {c[3] for c in ran} == {0, 1} and {c[0] for c in ran} == {1, 2, 4}
    assert any(c[1] == 64 for c in ran) == (D <= 64)
    assert any(c[2] == 2 for c in ran) == (D <= 64 and T % 64 == 0)


@pytest.mark.parametrize("D,Tq,Tk", [(128, 300, 1000), (64, 64, 2048), (32, 1, 777)])
def test_poison_continuation(D, Tq, Tk):
    B, Hq, Hkv = 1, 8, 2
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(B, Hq, Hkv, Tk, D, "bf16", seed=Tq))
    qn = q[:, :, -Tq:].contiguous()
    say(f"case poison fwd_kv D={D} Tq={Tq} Tk={Tk}")
    prod, pois = both(lambda: binding.attn_fwd_kv(qn, k, v, causal=True))
    same(prod, pois, f"fwd_kv D={D} Tq={Tq} Tk={Tk}")


@pytest.mark.parametrize("D", [32, 64, 128])
def test_poison_fp32(D):
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(1, 4, 2, 200, D, "fp32", seed=D))
    for causal in (True, False):
        say(f"case poison fp32 D={D} causal={causal}")
        prod, pois = both(lambda: binding.attn_fwd(q, k, v, causal=causal))
        same(prod, pois, f"fp32 D={D} causal={causal}")


@pytest.mark.parametrize("D", [32, 64, 128])
@pytest.mark.parametrize("T", [200, 512])
@pytest.mark.parametrize("causal", [True, False])
def test_poison_backward(D, T, causal):
    B, Hq, Hkv = 1, 8, 2
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=T + D))
    g = torch.Generator().manual_seed(T)
    do = torch.randn((B, Hq, T, D), generator=g).to(torch.bfloat16).to(DEV)
    out, lse = binding.attn_fwd(q, k, v, causal=causal)
    say(f"case poison bwd D={D} T={T} causal={causal}")
    prod, pois = both(lambda: binding.attn_bwd(q, k, v, out, lse, do, causal=causal))
    same(prod, pois, f"bwd D={D} T={T} causal={causal}")


# 576 dk/dv workgroups (one per KV head and 128-key tile), more than two per
# CU on 256 CUs: at D <= 64 the library runs its two-workgroups-per-CU dk/dv
# build here, and the one-step-late build on the grids above.
@pytest.mark.parametrize("D", [32, 64])
@pytest.mark.parametrize("causal", [True, False])
def test_poison_backward_large_grid(D, causal):
    B, Hq, Hkv, T = 8, 16, 8, 1100
    q, k, v = (t.to(DEV) for t in inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=T + D))
    g = torch.Generator().manual_seed(T)
    do = torch.randn((B, Hq, T, D), generator=g).to(torch.bfloat16).to(DEV)
    out, lse = binding.attn_fwd(q, k, v, causal=causal)
    say(f"case poison bwd large grid D={D} T={T} causal={causal}")
    prod, pois = both(lambda: binding.attn_bwd(q, k, v, out, lse, do, causal=causal))
    same(prod, pois, f"bwd large grid D={D} T={T} causal={causal}")


_rng = np.random.default_rng(9)
PAGED = [
    (9, 8, 2, 1, 128, 16, [1, 15, 16, 17, 100, 511, 512, 513, 3000], True),
    (6, 16, 4, 4, 64, 32, [0, 2, 4, 33, 1000, 2047], True),
    (5, 16, 2, 2, 32, 48, [1, 47, 48, 770, 1500], True),
    (4, 8, 8, 1, 128, 16, [7, 300, 301, 900], False),
    (70, 8, 2, 1, 64, 16, [int(x) for x in _rng.integers(0, 400, size=70)], True),
]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,D,bs,lens,causal", PAGED)
def test_poison_paged(B, Hq, Hkv, Tq, D, bs, lens, causal):
    q, kc, vc, table, cl = (t.to(DEV) for t in inputs.make_paged(
        B, Hq, Hkv, Tq, D, bs, context_lens=lens, spare=5, seed=B + D))
    say(f"case poison paged B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} D={D} bs={bs} causal={causal}")
    # rows that see no token give lse = -inf by contract
    prod, pois = both(lambda: binding.paged_decode(q, kc, vc, table, cl, causal=causal))
    same(prod, pois, f"paged D={D} bs={bs}", finite=False)
    assert torch.isfinite(pois[0]).all()

    def noalloc():
        o = torch.empty_like(q)
        l = torch.empty((B, Hq, Tq), device=DEV, dtype=torch.float32)
        binding.paged_decode_noalloc_into(q, kc, vc, table, cl, o, l, causal=causal)
        return o, l
    prod, pois = both(noalloc)
    same(prod, pois, f"paged noalloc D={D} bs={bs}", finite=False)
