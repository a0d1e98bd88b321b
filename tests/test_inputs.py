"""CPU tests of the seeded synthetic input generator."""
import numpy as np
import torch

from attention_flashattention_fwd_amd import inputs


def test_draws_are_seeded_and_ordered():
    q1, k1, v1 = inputs.draw_fp32(1, 2, 1, 8, 4, seed=0)
    q2, k2, v2 = inputs.draw_fp32(1, 2, 1, 8, 4, seed=0)
    assert np.array_equal(q1, q2) and np.array_equal(k1, k2) and np.array_equal(v1, v2)
    rng = np.random.default_rng(0)
    assert np.array_equal(q1, rng.standard_normal((1, 2, 8, 4), dtype=np.float32))
    assert np.array_equal(k1, rng.standard_normal((1, 1, 8, 4), dtype=np.float32))
    q3, _, _ = inputs.draw_fp32(1, 2, 1, 8, 4, seed=1)
    assert not np.array_equal(q1, q3)


def test_bf16_cast_is_round_to_nearest_even():
    x = np.array([1.0, 1.0 + 2.0 ** -8, 1.0 + 3 * 2.0 ** -8, -2.5], np.float32)
    t = torch.from_numpy(x).to(torch.bfloat16)
    b = inputs.bits(t)
    assert b.dtype == np.uint16
    # ties go to even: 1+2^-8 -> 1.0 ; 1+3*2^-8 -> 1+2^-6 (0x3F82)
    assert list(b) == [0x3F80, 0x3F80, 0x3F82, 0xC020]


def test_element_outliers_fraction():
    q, k, _ = inputs.draw_fp32(2, 4, 2, 512, 64, seed=0, outliers="elements")
    q0, k0, _ = inputs.draw_fp32(2, 4, 2, 512, 64, seed=0)
    ratio_q = (q != q0).mean()
    assert 0.008 < ratio_q < 0.012
    changed = q != q0
    assert np.array_equal(q[changed], q0[changed] * 8)
    assert 0.008 < (k != k0).mean() < 0.012


def test_row_outliers_scale_whole_rows():
    q, k, _ = inputs.draw_fp32(2, 4, 2, 2048, 16, seed=0, outliers="rows")
    q0, _, _ = inputs.draw_fp32(2, 4, 2, 2048, 16, seed=0)
    rows = (q != q0).any(-1)
    assert np.array_equal(q[rows], q0[rows] * 8)
    assert 0.006 < rows.mean() < 0.014


def test_workload_table():
    w = inputs.WORKLOADS["t16384_d128"]
    assert (w.B, w.Hq, w.Hkv, w.T, w.D, w.dtype, w.causal) == (1, 32, 8, 16384, 128, "bf16", True)
    assert abs(w.flops - 2.199e12) / 2.199e12 < 1e-3
    assert inputs.default_scale(128) == float(np.float32(1 / np.sqrt(128)))
    assert inputs.WORKLOADS["fp32_t64"].dtype == "fp32"


def test_kv_workload_counts_and_rows():
    """A continuation workload counts i + Tk - Tq + 1 visible keys for row i,
    reduces to the full count when Tq = Tk, and takes the last Tq query rows
    of the full draw."""
    w = inputs.KVWorkload("x", 1, 2, 1, 3, 5, 8)
    assert w.pairs == (2 + 1) + (2 + 2) + (2 + 3)   # Tk - Tq = 2
    full = inputs.KVWorkload("y", 2, 4, 2, 7, 7, 16)
    same = inputs.Workload("y", 2, 4, 2, 7, 16, "bf16", True)
    assert full.flops == same.pair_flops
    assert inputs.KVWorkload("z", 1, 2, 1, 3, 5, 8, causal=False).pairs == 15
    small = inputs.KVWorkload("s", 1, 2, 1, 4, 9, 8)
    q, k, v = inputs.make_kv_workload(small)
    qf, kf, vf = inputs.make_qkv(1, 2, 1, 9, 8, "bf16", 0)
    assert q.shape == (1, 2, 4, 8) and k.shape == (1, 1, 9, 8)
    assert torch.equal(q, qf[:, :, 5:]) and torch.equal(k, kf) and torch.equal(v, vf)


def test_paged_inputs_structure():
    """Every used block belongs to exactly one sequence, unused table entries
    are -1, lengths are drawn in range, and the draw is seeded."""
    q, kc, vc, table, lens = inputs.make_paged(6, 4, 2, 2, 32, 16, ctx_range=(1, 100), spare=5,
                                               max_blocks=7, seed=4)
    assert q.shape == (6, 4, 2, 32) and kc.shape == vc.shape and kc.shape[1:] == (2, 16, 32)
    assert table.shape == (6, 7) and table.dtype == torch.int32 and lens.dtype == torch.int32
    n = lens.numpy().astype(np.int64)
    assert ((1 <= n) & (n <= 100)).all()
    nblk = -(-n // 16)
    used = np.concatenate([table[b, :nblk[b]].numpy() for b in range(6)])
    assert len(set(used.tolist())) == used.size == nblk.sum()
    assert kc.shape[0] == used.size + 5 and (used >= 0).all() and (used < kc.shape[0]).all()
    assert all((table[b, nblk[b]:] == -1).all() for b in range(6))
    again = inputs.make_paged(6, 4, 2, 2, 32, 16, ctx_range=(1, 100), spare=5, max_blocks=7,
                              seed=4)
    assert all(torch.equal(a, b) for a, b in zip((q, kc, vc, table, lens), again))


def test_paged_workload_and_bytes():
    w = inputs.PAGED_WORKLOADS["decode_b64_ctx16k_d128"]
    assert (w.B, w.Hq, w.Hkv, w.Tq, w.D, w.block_size) == (64, 32, 8, 1, 128, 16)
    assert w.max_blocks == 1024
    # one sequence of 17 tokens, Hkv = 2, D = 8, blocks of 16: K and V rows,
    # q and out (bf16), lse (fp32), two table entries and one length
    got = inputs.paged_bytes([17], Hq=4, Hkv=2, Tq=1, D=8, block_size=16)
    assert got == 2 * 2 * 2 * 8 * 17 + 2 * 2 * 4 * 8 + 4 * 4 + 4 * 2 + 4
