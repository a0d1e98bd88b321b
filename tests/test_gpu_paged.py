"""GPU parity of tessera_paged_decode (attention decode over a block-paged KV
cache) against the fp64 oracle, through the C ABI.  Same bar as the forward:
bf16 max-abs <= 2e-2 and mean-abs <= 2e-3 for O and for the finite lse; rows
that see no token must give exactly O = 0 and lse = -inf."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from attention_flashattention_fwd_amd import binding, inputs
from tests.test_gpu_parity import BF16_MAX, BF16_MEAN, say

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda:0")


def to_dev(*ts):
    return tuple(t.to(DEV) for t in ts)


def run_paged(q, kc, vc, table, lens, causal, scale):
    out, lse = binding.paged_decode(*to_dev(q, kc, vc, table, lens), causal=causal, scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def reference(q, kc, vc, table, lens, causal, scale):
    return oracle.paged_decode(inputs.bits(q), inputs.bits(kc), inputs.bits(vc), table.numpy(),
                               lens.numpy(), causal, scale)


def check_paged(o, l, O_ref, l_ref, what=""):
    empty = np.isneginf(l_ref)
    assert np.isfinite(o).all(), f"non-finite O {what}"
    assert np.array_equal(np.isneginf(l), empty), f"-inf lse rows differ {what}"
    assert np.isfinite(l[~empty]).all(), f"non-finite lse {what}"
    assert np.all(o[empty] == 0.0), f"rows that see no token must be 0 {what}"
    eo = np.abs(o - O_ref)
    el = np.abs(l[~empty] - l_ref[~empty]) if (~empty).any() else np.zeros(1)
    stats = (f"{what} O max {eo.max():.3e} mean {eo.mean():.3e} | lse max {el.max():.3e} "
             f"mean {el.mean():.3e} | empty rows {int(empty.sum())}")
    say(stats)
    assert eo.max() <= BF16_MAX and eo.mean() <= BF16_MEAN, stats
    assert el.max() <= BF16_MAX and el.mean() <= BF16_MEAN, stats


# (B, Hq, Hkv, Tq, D, block_size, lengths, causal).  The lengths cross block
# and tile (32 keys) boundaries and the boundaries of the waves' shares (at
# these sizes most waves hold one tile, so a long sequence is cut into many
# pieces: 94 for the 3000-token one, more than the merge's 64 at a time), and
# include empty sequences and sequences shorter than Tq.  More than 64
# sequences give each lane several sequences to count; a single long
# sequence is cut among all waves of its head.
_rng = np.random.default_rng(5)
MANY_100 = [int(x) for x in _rng.integers(0, 600, size=100)]
MANY_100[7] = MANY_100[64] = MANY_100[99] = 0
MANY_300 = [int(x) for x in _rng.integers(0, 200, size=300)]
MANY_300[0] = MANY_300[150] = 0
CASES = [
    (9, 8, 2, 1, 128, 16, [1, 15, 16, 17, 100, 511, 512, 513, 3000], True),
    (6, 16, 4, 4, 64, 32, [0, 2, 4, 33, 1000, 2047], True),
    (5, 16, 2, 2, 32, 48, [1, 47, 48, 770, 1500], True),
    (3, 32, 4, 4, 128, 16, [3, 260, 1900], True),        # 32 query rows per KV head
    (4, 4, 1, 3, 64, 64, [0, 1, 5, 4100], True),         # MQA, a 17-split sequence
    (4, 8, 8, 1, 128, 16, [7, 300, 301, 900], False),
    (3, 8, 2, 8, 64, 16, [5, 64, 700], False),           # non-causal, n < Tq included
    (100, 8, 2, 1, 64, 16, MANY_100, True),               # two sequences per lane
    (300, 4, 1, 2, 32, 16, MANY_300, True),               # five per lane, MQA
    (1, 32, 8, 1, 128, 16, [16000], True),                # one sequence, 192 pieces per head
]


@pytest.mark.parametrize("B,Hq,Hkv,Tq,D,bs,lens,causal", CASES)
def test_paged_shapes(B, Hq, Hkv, Tq, D, bs, lens, causal):
    q, kc, vc, table, cl = inputs.make_paged(B, Hq, Hkv, Tq, D, bs, context_lens=lens,
                                             spare=7, seed=sum(lens) + D)
    scale = inputs.default_scale(D)
    say(f"case paged B={B} Hq={Hq} Hkv={Hkv} Tq={Tq} D={D} bs={bs} lens={lens} causal={causal} "
        f"workspace={binding.paged_workspace_bytes(B, Hq, Hkv, Tq, D, bs, table.shape[1])}")
    o, l = run_paged(q, kc, vc, table, cl, causal, scale)
    O_ref, l_ref = reference(q, kc, vc, table, cl, causal, scale)
    check_paged(o, l, O_ref, l_ref)


def test_paged_scale_sign_and_zero():
    q, kc, vc, table, cl = inputs.make_paged(3, 8, 2, 2, 64, 16, context_lens=[1, 40, 700],
                                             seed=11)
    for scale in (-0.2, 0.0, 0.5, 8.0, -8.0):
        say(f"case paged scale={scale}")
        o, l = run_paged(q, kc, vc, table, cl, True, scale)
        O_ref, l_ref = reference(q, kc, vc, table, cl, True, scale)
        check_paged(o, l, O_ref, l_ref, f"scale={scale}")


def test_paged_all_sequences_empty():
    q, kc, vc, table, cl = inputs.make_paged(3, 8, 2, 2, 128, 16, context_lens=[0, 0, 0],
                                             spare=2, max_blocks=40, seed=12)
    say("case paged all empty")
    o, l = run_paged(q, kc, vc, table, cl, True, 0.1)
    assert np.all(o == 0.0) and np.all(np.isneginf(l))


@pytest.mark.parametrize("D,bs", [(128, 16), (64, 32), (32, 48)])
def test_paged_nan_in_rows_no_sequence_owns(D, bs):
    """Cache rows that no sequence owns -- those past a sequence's length in
    its last block, and the spare blocks -- hold NaN.  The kernel never reads
    them, so the output equals the oracle's on the finite cache and the
    kernel's own output with finite values there, bit for bit."""
    lens = [1, 15, 17, 100, 333, 0, 1000]
    q, kc, vc, table, cl = inputs.make_paged(7, 8, 2, 2, D, bs, context_lens=lens, spare=3,
                                             seed=21 + D)
    owned = torch.zeros((kc.shape[0], bs), dtype=torch.bool)
    for b, n in enumerate(lens):
        for t in range(n):
            owned[int(table[b, t // bs]), t % bs] = True
    assert (~owned).any()
    kn, vn = kc.clone(), vc.clone()
    for c in (kn, vn):
        c.permute(0, 2, 1, 3)[~owned] = float("nan")
    scale = inputs.default_scale(D)
    say(f"case paged NaN outside the sequences D={D} bs={bs} unowned rows={int((~owned).sum())}")
    o, l = run_paged(q, kn, vn, table, cl, True, scale)
    O_ref, l_ref = reference(q, kc, vc, table, cl, True, scale)
    check_paged(o, l, O_ref, l_ref, "NaN outside the sequences")
    o2, l2 = run_paged(q, kc, vc, table, cl, True, scale)
    assert np.array_equal(o, o2) and np.array_equal(l, l2)


def test_paged_bad_table_entry_and_length_give_nan():
    """A sequence with a table entry out of range, or a length past the
    table, gets NaN everywhere; the other sequences are unaffected."""
    lens = [300, 900, 50, 600]
    q, kc, vc, table, cl = inputs.make_paged(4, 8, 2, 1, 64, 16, context_lens=lens, spare=3,
                                             seed=13)
    good_o, good_l = reference(q, kc, vc, table, cl, True, 0.125)
    bad_table = table.clone()
    bad_table[0, 3] = kc.shape[0]        # sequence 0, in its first split
    bad_table[1, 40] = -5                # sequence 1, in its third split
    bad_lens = cl.clone()
    bad_lens[2] = table.shape[1] * 16 + 1
    say("case paged bad device data")
    o, l = run_paged(q, kc, vc, bad_table, bad_lens, True, 0.125)
    for b in range(3):
        assert np.isnan(o[b]).all() and np.isnan(l[b]).all(), b
    check_paged(o[3:], l[3:], good_o[3:], good_l[3:], "untouched sequence")


def test_paged_matches_contiguous_kv_path():
    """The same rows through tessera_attn_fwd_kv on the gathered cache."""
    lens = [40, 1000, 333]
    q, kc, vc, table, cl = inputs.make_paged(3, 8, 2, 3, 128, 16, context_lens=lens, seed=14)
    o, l = run_paged(q, kc, vc, table, cl, True, 0.09)
    for b, n in enumerate(lens):
        t = torch.arange(n)
        rows = table[b].long()[t // 16] * 16 + t % 16
        k = kc.permute(1, 0, 2, 3).reshape(2, -1, 128)[:, rows][None].contiguous()
        v = vc.permute(1, 0, 2, 3).reshape(2, -1, 128)[:, rows][None].contiguous()
        ok, lk = binding.attn_fwd_kv(*to_dev(q[b:b + 1], k, v), causal=True, scale=0.09)
        torch.cuda.synchronize()
        eo = np.abs(o[b] - ok[0].float().cpu().numpy()).max()
        el = np.abs(l[b] - lk[0].cpu().numpy()).max()
        say(f"sequence {b} n={n}: paged vs contiguous O {eo:.3e} lse {el:.3e}")
        assert eo <= BF16_MAX and el <= BF16_MAX


def test_paged_workspace_reuse_and_stream():
    """Two calls in a row on one workspace (the second smaller), on a side
    stream, each equal to a fresh call's bits."""
    big = inputs.make_paged(4, 8, 2, 2, 64, 16, context_lens=[900, 20, 2000, 513], seed=15)
    small = inputs.make_paged(2, 8, 2, 2, 64, 16, context_lens=[700, 1], seed=16)
    nbytes = binding.paged_workspace_bytes(4, 8, 2, 2, 64, 16, big[3].shape[1])
    assert nbytes > 0
    ws = torch.full((nbytes,), 0x7f, dtype=torch.uint8, device=DEV)
    side = torch.cuda.Stream(DEV)
    for case in (big, small):
        q, kc, vc, table, cl = to_dev(*case)
        out = torch.empty_like(q)
        lse = torch.empty(q.shape[:3], dtype=torch.float32, device=DEV)
        side.wait_stream(torch.cuda.current_stream(DEV))
        with torch.cuda.stream(side):
            binding.paged_decode_into(q, kc, vc, table, cl, out, lse, ws, True, 0.125,
                                      stream=side)
        side.synchronize()
        o2, l2 = binding.paged_decode(q, kc, vc, table, cl, True, 0.125)
        torch.cuda.synchronize()
        assert torch.equal(out, o2) and torch.equal(lse, l2)


def test_paged_serving_workload_sampled():
    """The 64-sequence serving batch at full size (the bench's launch):
    eight sequences, the longest and shortest among them, checked whole
    against the oracle."""
    w = inputs.PAGED_WORKLOADS["decode_b64_ctx16k_d128"]
    q, kc, vc, table, cl = inputs.make_paged_workload(w)
    say(f"case paged workload {w.name}: {w.describe()}, cache {2 * kc.numel() * 2 / 1e9:.2f} GB")
    o, l = run_paged(q, kc, vc, table, cl, w.causal, w.scale)
    n = cl.numpy()
    pick = sorted({int(n.argmax()), int(n.argmin()), 0, 1, 17, 31, 32, 63})
    sub = np.array(pick)
    O_ref, l_ref = oracle.paged_decode(inputs.bits(q[sub]), inputs.bits(kc), inputs.bits(vc),
                                       table.numpy()[sub], n[sub], w.causal, w.scale)
    check_paged(o[sub], l[sub], O_ref, l_ref, f"sequences {pick}")


def test_paged_cache_offsets_past_int32():
    """K/V caches of 140000 blocks x 8 KV heads x 16 x 128 elements (more than
    2^31), with every table entry in the blocks past 2^31 elements.  The oracle
    takes the same rows, gathered into a small cache under a renumbered table
    (its answer does not depend on where blocks sit)."""
    B, Hq, Hkv, Tq, D, bs, nblk, max_blocks = 2, 32, 8, 1, 128, 16, 140000, 64
    first_high = 2 ** 31 // (Hkv * bs * D)                 # first block past 2^31 elements
    assert nblk * Hkv * bs * D > 2 ** 31 and first_high == 131072
    dev = torch.device("cuda:0")
    say(f"case paged int32-overflowing cache offsets blocks={nblk} Hkv={Hkv} bs={bs} D={D}")
    q, kc, vc = inputs.randn_on_device(((B, Hq, Tq, D), (nblk, Hkv, bs, D), (nblk, Hkv, bs, D)),
                                       seed=24, device=dev)
    lens = torch.tensor([700, max_blocks * bs], dtype=torch.int32)
    rng = np.random.default_rng(24)
    ids = rng.choice(np.arange(first_high, nblk), size=B * max_blocks, replace=False)
    table = torch.from_numpy(ids.reshape(B, max_blocks).astype(np.int32))
    scale = inputs.default_scale(D)
    out, lse = binding.paged_decode(q, kc, vc, table.to(dev), lens.to(dev), causal=True,
                                    scale=scale)
    torch.cuda.synchronize()
    used = torch.from_numpy(ids.astype(np.int64)).to(dev)
    kc_small, vc_small = kc[used].cpu(), vc[used].cpu()
    table_small = np.arange(B * max_blocks, dtype=np.int32).reshape(B, max_blocks)
    O_ref, l_ref = oracle.paged_decode(inputs.bits(q.cpu()), inputs.bits(kc_small),
                                       inputs.bits(vc_small), table_small, lens.numpy(), True,
                                       scale)
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    check_paged(o, l, O_ref, l_ref, "high blocks")
    del q, kc, vc, out, lse, used
    torch.cuda.empty_cache()
