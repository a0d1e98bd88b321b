"""GPU test of tessera_paged_decode_noalloc, the paged decode for callers that
cannot allocate: its split partials use the library's fixed per-GPU scratch
buffer instead of a caller workspace.  Through the C ABI it must give what
tessera_paged_decode gives with a workspace of its own (the same kernels and
the same split plan, so the same bits), on consecutive calls of different
sizes that share the buffer, and allocate nothing."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from attention_flashattention_fwd_amd import binding, inputs
from tests.test_gpu_paged import check_paged
from tests.test_gpu_parity import say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def decode_both(q, kc, vc, table, lens, causal, scale):
    """(out, lse) from the workspace entry point and from the allocation-free
    one, on the same device inputs; the second call allocates nothing."""
    q, kc, vc, table, lens = (t.to(DEV) for t in (q, kc, vc, table, lens))
    ref_out, ref_lse = binding.paged_decode(q, kc, vc, table, lens, causal=causal, scale=scale)
    out = torch.full_like(q, float("nan"))
    lse = torch.full(ref_lse.shape, float("nan"), dtype=torch.float32, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated(DEV)
    binding.paged_decode_noalloc_into(q, kc, vc, table, lens, out, lse, causal=causal,
                                      scale=scale)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated(DEV) == before
    return (ref_out, ref_lse), (out, lse)


def check_same_and_oracle(pw_args, causal, pick, what):
    q, kc, vc, table, lens = pw_args
    B, Hq, Tq, D = q.shape
    scale = inputs.default_scale(D)
    nws = binding.paged_workspace_bytes(B, Hq, kc.shape[1], Tq, D, kc.shape[2], table.shape[1])
    say(f"case {what}: B={B} Hq={Hq} Hkv={kc.shape[1]} Tq={Tq} D={D} "
        f"block_size={kc.shape[2]} max_blocks={table.shape[1]} workspace {nws} bytes")
    assert 0 < nws <= binding.paged_scratch_limit()   # the split path, inside the limit
    (ro, rl), (o, l) = decode_both(q, kc, vc, table, lens, causal, scale)
    assert torch.equal(o, ro) and torch.equal(l, rl), "no-alloc differs from the workspace call"
    O_ref, l_ref = oracle.paged_decode(inputs.bits(q[pick]), inputs.bits(kc), inputs.bits(vc),
                                       table.numpy()[pick], lens.numpy()[pick], causal, scale)
    got_o = o[torch.from_numpy(pick).to(DEV)].float().cpu().numpy().astype(np.float64)
    got_l = l[torch.from_numpy(pick).to(DEV)].cpu().numpy().astype(np.float64)
    say(f"{what}: equal to the workspace call; sequences {pick.tolist()} against the oracle:")
    check_paged(got_o, got_l, O_ref, l_ref, what)


def test_noalloc_matches_the_workspace_entry_on_two_calls():
    # first the serving batch (17 MB of partials), then a smaller decode whose
    # partials cover only the start of the buffer the first call filled
    pw = inputs.PAGED_WORKLOADS["decode_b64_ctx16k_d128"]
    big = inputs.make_paged_workload(pw)
    n = big[4].numpy()
    check_same_and_oracle(big, pw.causal, np.array(sorted({int(n.argmax()), 0, pw.B - 1})),
                          "serving batch")
    small = inputs.make_paged(6, 16, 4, 2, 64, 16, context_lens=[0, 3, 300, 1000, 2500, 4000],
                              max_blocks=256, seed=31)
    check_same_and_oracle(small, True, np.arange(6), "smaller decode after it")


def test_noalloc_rejects_what_exceeds_the_scratch():
    # 32 query rows per KV head: 8 x 256 slots of 32 rows, 34 MB of workspace
    q = torch.zeros(64, 256, 1, 128, dtype=torch.bfloat16, device=DEV)
    kc = torch.zeros(8, 8, 16, 128, dtype=torch.bfloat16, device=DEV)
    table = torch.zeros(64, 4096, dtype=torch.int32, device=DEV)
    lens = torch.zeros(64, dtype=torch.int32, device=DEV)
    out, lse = torch.empty_like(q), torch.empty(64, 256, 1, device=DEV)
    assert binding.paged_workspace_bytes(64, 256, 8, 1, 128, 16, 4096) > binding.paged_scratch_limit()
    with pytest.raises(RuntimeError, match="scratch"):
        binding.paged_decode_noalloc_into(q, kc, kc, table, lens, out, lse)
