"""Pins of the fp64 paged-decode oracle to facts other than itself.

  * the contiguous continuation oracle (attn_fwd_kv, itself pinned): the K/V
    rows of each sequence gathered block by block into one [Hkv, n, D] tensor
    give the same rows of O and lse;
  * torch's scaled_dot_product_attention in float64 on the CPU, over K/V
    gathered a second, independent way (one flat index per token), with an
    explicit bottom-right-aligned mask;
  * invariants of the paging: relabelling the physical blocks, or storing the
    same tokens in blocks of another size, changes no bit;
  * closed forms: a row that sees no token gives O = 0 and lse = -inf; with
    identical value rows O equals that row; with Tq = 1 the causal and the
    full result agree (the newest token sees every cached one).
"""
from __future__ import annotations

import math

import numpy as np
import torch

from tests.oracle_pins import as_dtype, fp32, values


def rand_paged(B, Hq, Hkv, Tq, D, block_size, lens, seed, spare=3):
    """A paged cache with randomly placed blocks (numpy draws only)."""
    rng = np.random.default_rng(seed)
    lens = np.asarray(lens, dtype=np.int32)
    nblk = -(-lens // block_size)
    max_blocks = max(1, int(nblk.max()) + 1)
    num_blocks = int(nblk.sum()) + spare
    perm = rng.permutation(num_blocks).astype(np.int32)
    table = np.full((B, max_blocks), -1, np.int32)
    at = 0
    for b in range(B):
        table[b, :nblk[b]] = perm[at:at + nblk[b]]
        at += int(nblk[b])
    q = as_dtype(rng.standard_normal((B, Hq, Tq, D)), "bf16")
    kc = as_dtype(rng.standard_normal((num_blocks, Hkv, block_size, D)), "bf16")
    vc = as_dtype(rng.standard_normal((num_blocks, Hkv, block_size, D)), "bf16")
    return q, kc, vc, table, lens


def gather_by_blocks(cache, table_row, n):
    """[Hkv, n, D]: the first n tokens of one sequence, block after block."""
    block_size = cache.shape[2]
    parts = [cache[table_row[j]] for j in range(-(-n // block_size))]
    if not parts:
        return np.zeros((cache.shape[1], 0, cache.shape[3]), cache.dtype)
    return np.concatenate(parts, axis=1)[:, :n]


# Shapes: (B, Hq, Hkv, Tq, D, block_size, lengths).  Lengths cover an empty
# sequence, fewer tokens than new rows, block boundaries and ragged ends.
CASES = [
    (4, 4, 2, 1, 8, 16, [0, 1, 16, 37]),
    (3, 6, 2, 3, 16, 16, [2, 33, 64]),
    (2, 4, 4, 4, 8, 32, [70, 4]),
    (3, 8, 1, 2, 32, 48, [1, 95, 49]),
]


def pin_paged_equals_contiguous(lib):
    for n_case, (B, Hq, Hkv, Tq, D, bs, lens) in enumerate(CASES):
        q, kc, vc, table, lens = rand_paged(B, Hq, Hkv, Tq, D, bs, lens, seed=600 + n_case)
        scale = fp32(1.0 / math.sqrt(D))
        for causal in (True, False):
            O, lse = lib.paged_decode(q, kc, vc, table, lens, causal, scale)
            for b in range(B):
                n = int(lens[b])
                first = max(0, Tq - n) if causal else (Tq if n == 0 else 0)
                assert np.all(O[b, :, :first] == 0.0), (n_case, b, causal)
                assert np.all(lse[b, :, :first] == -np.inf), (n_case, b, causal)
                if first == Tq:
                    continue
                k = gather_by_blocks(kc, table[b], n)[None]
                v = gather_by_blocks(vc, table[b], n)[None]
                qb = np.ascontiguousarray(q[b:b + 1, :, first:])
                Ok, lk = lib.attn_fwd_kv(qb, np.ascontiguousarray(k), np.ascontiguousarray(v),
                                         causal, scale)
                assert np.abs(O[b:b + 1, :, first:] - Ok).max() <= 1e-12, (n_case, b, causal)
                assert np.abs(lse[b:b + 1, :, first:] - lk).max() <= 1e-12, (n_case, b, causal)


def pin_paged_torch_sdpa(lib):
    for n_case, (B, Hq, Hkv, Tq, D, bs, lens) in enumerate(CASES):
        q, kc, vc, table, lens = rand_paged(B, Hq, Hkv, Tq, D, bs, lens, seed=700 + n_case)
        scale = fp32(0.5 + 0.1 * n_case)
        O, lse = lib.paged_decode(q, kc, vc, table, lens, True, scale)
        G = Hq // Hkv
        kflat = torch.from_numpy(values(kc)).permute(1, 0, 2, 3).reshape(Hkv, -1, D)
        vflat = torch.from_numpy(values(vc)).permute(1, 0, 2, 3).reshape(Hkv, -1, D)
        for b in range(B):
            n = int(lens[b])
            if n == 0:
                continue
            t = torch.arange(n)
            flat = torch.from_numpy(table[b]).long()[t // bs] * bs + t % bs
            k = kflat[:, flat].repeat_interleave(G, dim=0)
            v = vflat[:, flat].repeat_interleave(G, dim=0)
            qt = torch.from_numpy(values(q[b]))
            visible = t[None, :] <= torch.arange(Tq)[:, None] + (n - Tq)
            seen = visible.any(dim=1)
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt[:, seen], k, v, attn_mask=visible[seen], scale=scale)
            assert np.abs(O[b][:, seen.numpy()] - ref.numpy()).max() <= 1e-12, (n_case, b)
            s = ((qt @ k.transpose(-1, -2)) * scale).masked_fill(~visible, float("-inf"))
            ref_lse = torch.logsumexp(s, dim=-1).numpy()
            assert np.array_equal(np.isinf(lse[b]), np.isinf(ref_lse)), (n_case, b)
            fin = np.isfinite(ref_lse)
            assert np.abs(lse[b][fin] - ref_lse[fin]).max() <= 1e-12, (n_case, b)


def repack(cache, table, lens, new_bs, seed):
    """The same tokens stored in blocks of new_bs rows at random places."""
    B = table.shape[0]
    Hkv, bs, D = cache.shape[1], cache.shape[2], cache.shape[3]
    rng = np.random.default_rng(seed)
    nblk = -(-lens // new_bs)
    num_blocks = int(nblk.sum()) + 2
    perm = rng.permutation(num_blocks).astype(np.int32)
    out = np.zeros((num_blocks, Hkv, new_bs, D), cache.dtype)
    new_table = np.full((B, max(1, int(nblk.max()))), -1, np.int32)
    at = 0
    for b in range(B):
        n = int(lens[b])
        rows = gather_by_blocks(cache, table[b], n)
        for j in range(nblk[b]):
            blk = perm[at + j]
            new_table[b, j] = blk
            part = rows[:, j * new_bs:(j + 1) * new_bs]
            out[blk, :, :part.shape[1]] = part
        at += int(nblk[b])
    return out, new_table


def pin_paged_layout_invariance(lib):
    B, Hq, Hkv, Tq, D, bs, lens = 3, 4, 2, 2, 16, 16, [5, 40, 64]
    q, kc, vc, table, lens = rand_paged(B, Hq, Hkv, Tq, D, bs, lens, seed=71)
    O, lse = lib.paged_decode(q, kc, vc, table, lens, True, 0.25)
    # Relabel the physical blocks.
    rng = np.random.default_rng(5)
    relabel = rng.permutation(kc.shape[0]).astype(np.int32)
    kc2, vc2 = np.empty_like(kc), np.empty_like(vc)
    kc2[relabel], vc2[relabel] = kc, vc
    table2 = np.where(table >= 0, relabel[np.maximum(table, 0)], -1).astype(np.int32)
    O2, lse2 = lib.paged_decode(q, kc2, vc2, table2, lens, True, 0.25)
    assert np.array_equal(O, O2) and np.array_equal(lse, lse2)
    # Other block sizes.
    for new_bs in (1, 3, 32):
        kc3, table3 = repack(kc, table, lens, new_bs, seed=new_bs)
        vc3, _ = repack(vc, table, lens, new_bs, seed=new_bs)
        O3, lse3 = lib.paged_decode(q, kc3, vc3, table3, lens, True, 0.25)
        assert np.array_equal(O, O3) and np.array_equal(lse, lse3), new_bs


def pin_paged_closed_forms(lib):
    B, Hq, Hkv, Tq, D, bs, lens = 3, 4, 2, 3, 8, 16, [0, 2, 29]
    q, kc, vc, table, lens = rand_paged(B, Hq, Hkv, Tq, D, bs, lens, seed=72)
    # No visible token: sequence 0 entirely, row 0 of sequence 1 (2 tokens, 3 rows).
    O, lse = lib.paged_decode(q, kc, vc, table, lens, True, 0.3)
    assert np.all(O[0] == 0.0) and np.all(lse[0] == -np.inf)
    assert np.all(O[1, :, 0] == 0.0) and np.all(lse[1, :, 0] == -np.inf)
    assert np.all(np.isfinite(lse[1, :, 1:])) and np.all(np.isfinite(lse[2]))
    # Identical value rows within each KV head: O is that row wherever a token is seen.
    row = as_dtype(np.arange(Hkv * D, dtype=np.float32).reshape(Hkv, 1, D) / 7.0, "bf16")
    vsame = np.ascontiguousarray(np.broadcast_to(row[None], vc.shape))
    O, lse = lib.paged_decode(q, kc, vsame, table, lens, True, 0.3)
    expect = np.repeat(values(row)[:, 0], Hq // Hkv, axis=0)   # [Hq, D]
    for b, i in ((1, 1), (1, 2), (2, 0), (2, 2)):
        assert np.abs(O[b, :, i] - expect).max() <= 1e-12, (b, i)
    # One new token per sequence: it sees every cached token with or without the mask.
    q1 = np.ascontiguousarray(q[:, :, :1])
    Oc, lc = lib.paged_decode(q1, kc, vc, table, lens, True, 0.3)
    Of, lf = lib.paged_decode(q1, kc, vc, table, lens, False, 0.3)
    assert np.array_equal(Oc, Of) and np.array_equal(lc, lf)


ALL_PAGED_PINS = [pin_paged_equals_contiguous, pin_paged_torch_sdpa, pin_paged_layout_invariance,
                  pin_paged_closed_forms]
