"""GPU parity: the HIP path (through the C ABI) against the fp64 CPU oracle.

Bar: bf16 inputs -- max-abs <= 2e-2 and mean-abs <= 2e-3, separately for O and
lse; fp32 inputs -- max-abs <= 1e-4.  Small shapes compare every element; the
full-size workloads compare sampled rows (the oracle computes them one by one)
and check properties that hold at any size on every row.
"""
from __future__ import annotations

import math

import numpy as np
import pytest
import torch

import oracle
from attention_flashattention_fwd_amd import binding, inputs

pytestmark = pytest.mark.gpu

BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4


def say(*msg):
    print(*msg, flush=True)


def run_gpu(q, k, v, causal, scale):
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out, lse = binding.attn_fwd(qd, kd, vd, causal=causal, scale=scale)
    torch.cuda.synchronize()
    return out.float().cpu().numpy().astype(np.float64), lse.cpu().numpy().astype(np.float64)


def check_close(o, l, O_ref, l_ref, dtype, what=""):
    assert np.isfinite(o).all() and np.isfinite(l).all(), f"non-finite output {what}"
    eo, el = np.abs(o - O_ref), np.abs(l - l_ref)
    stats = f"{what} O max {eo.max():.3e} mean {eo.mean():.3e} | lse max {el.max():.3e} mean {el.mean():.3e}"
    say(stats)
    if dtype == "bf16":
        assert eo.max() <= BF16_MAX and eo.mean() <= BF16_MEAN, stats
        assert el.max() <= BF16_MAX and el.mean() <= BF16_MEAN, stats
    else:
        assert eo.max() <= F32_MAX and el.max() <= F32_MAX, stats


def full_case(B, Hq, Hkv, T, D, dtype, causal, scale=None, seed=0, outliers=""):
    q, k, v = inputs.make_qkv(B, Hq, Hkv, T, D, dtype, seed, outliers)
    scale = inputs.default_scale(D) if scale is None else scale
    say(f"case B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} {dtype} causal={causal} scale={scale}")
    o, l = run_gpu(q, k, v, causal, scale)
    O_ref, l_ref = oracle.attn_fwd(inputs.bits(q), inputs.bits(k), inputs.bits(v), causal, scale)
    check_close(o, l, O_ref, l_ref, dtype)
    return q, k, v, o, l


def test_the_native_library_is_loaded():
    lib = binding.lib()
    assert lib._name == str(binding.library_path())
    assert binding.library_path().parent.name == "attention_flashattention_fwd_amd"


# -- the two small workloads, every element --------------------------------
def test_fp32_t64_workload():
    w = inputs.WORKLOADS["fp32_t64"]
    full_case(w.B, w.Hq, w.Hkv, w.T, w.D, w.dtype, w.causal)


def test_tiny_t128_workload():
    w = inputs.WORKLOADS["tiny_t128"]
    q, k, v, o, l = full_case(w.B, w.Hq, w.Hkv, w.T, w.D, w.dtype, w.causal)
    # causal row 0 sees only key 0: p = 1 exactly, so O = V[0] bit for bit
    G = w.Hq // w.Hkv
    v0 = np.repeat(v[:, :, 0].float().numpy(), G, axis=1)
    assert np.array_equal(o[:, :, 0], v0)


# -- edge shapes, every element -----------------------------------------------
EDGE = [
    # B, Hq, Hkv, T, D, causal
    (1, 4, 1, 1, 64, True),       # one row
    (1, 4, 4, 7, 32, True),       # MHA, T below one tile
    (3, 4, 2, 17, 64, False),
    (2, 8, 2, 65, 128, True),     # one key past a tile
    (1, 8, 1, 130, 64, True),     # MQA (G=8: two workgroups per query tile)
    (2, 6, 2, 200, 32, True),     # G=3: one head per workgroup, eight query blocks
    (1, 12, 2, 333, 64, False),   # G=6
    (1, 4, 4, 1000, 128, True),   # MHA, ragged, several tiles
    (2, 4, 1, 1000, 64, False),
    (1, 16, 4, 257, 32, True),
    (1, 32, 1, 300, 128, True),   # G=32: eight head slots per KV head
    (2, 10, 2, 150, 64, True),    # G=5: one head per workgroup
    (1, 14, 2, 100, 32, False),   # G=7
    (2, 8, 2, 777, 64, False),    # two query blocks per wave, ragged
]


@pytest.mark.parametrize("B,Hq,Hkv,T,D,causal", EDGE)
def test_edge_shapes_bf16(B, Hq, Hkv, T, D, causal):
    full_case(B, Hq, Hkv, T, D, "bf16", causal, seed=T)


# T a multiple of the 64-key tile: the kernel variant without the row clamp on
# K/V loads, with 1..9 tiles so that every position of the four-deep LDS ring
# ends a run, and each head grouping (G = 4, 3, 6, 1 and 2).
ALIGNED = [
    (1, 8, 2, 64, 128, True),     # one tile
    (2, 8, 2, 128, 64, True),
    (1, 4, 1, 192, 32, True),
    (1, 8, 2, 256, 128, False),
    (2, 6, 2, 320, 64, True),     # G=3
    (1, 12, 2, 384, 128, True),   # G=6
    (1, 4, 4, 576, 64, False),    # MHA
    (1, 4, 2, 448, 32, False),
]


@pytest.mark.parametrize("B,Hq,Hkv,T,D,causal", ALIGNED)
def test_aligned_shapes_bf16(B, Hq, Hkv, T, D, causal):
    full_case(B, Hq, Hkv, T, D, "bf16", causal, seed=T + 1)


# D = 64 grids of 2048 or more workgroups (query tiles x B x Hkv) with T a
# multiple of 64 run two workgroups per CU, a kernel build of their own; a
# ragged T of that size takes the one-workgroup build.  Each is compared
# element by element.
PAIRED = [
    (128, 32, 8, 128, 64, True),    # 2 query tiles x 1024 = 2048 workgroups
    (128, 16, 16, 128, 64, False),  # MHA: 256-row tiles, 1 x 2048
    (86, 32, 8, 130, 64, True),     # 3 x 688, ragged: one workgroup per CU
]


@pytest.mark.parametrize("B,Hq,Hkv,T,D,causal", PAIRED)
def test_two_workgroups_per_cu_shapes(B, Hq, Hkv, T, D, causal):
    full_case(B, Hq, Hkv, T, D, "bf16", causal, seed=B + T)


# Grids with at least four work items (query tile x KV head x head slot) per
# workgroup the GPU holds at once run as persistent launches that take items
# from per-XCD queues.  Each case below has more than 1024 items (four per CU
# on 256 CUs); every element is compared, and repeated calls on one stream and
# calls on two streams at once must give the same bits (each launch resets
# its queue counters, which are kept per stream).
PERSISTENT = [
    (8, 16, 4, 2112, 128, True),   # 1056 items
    (8, 16, 4, 2100, 128, True),   # ragged
    (8, 16, 4, 2112, 64, True),    # one workgroup per CU at D = 64
    (8, 16, 4, 2100, 64, True),    # ragged
    (128, 8, 8, 300, 64, False),   # two query blocks per wave, 1024 items
    (4, 32, 8, 2100, 32, True),    # 1056 items
    (128, 8, 8, 64, 128, True),    # 1024 one-tile items
]


@pytest.mark.parametrize("B,Hq,Hkv,T,D,causal", PERSISTENT)
def test_persistent_launch_shapes(B, Hq, Hkv, T, D, causal):
    q, k, v, o, l = full_case(B, Hq, Hkv, T, D, "bf16", causal, seed=T + B)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    outs = [binding.attn_fwd(qd, kd, vd, causal=causal) for _ in range(3)]
    torch.cuda.synchronize()
    ref_o = torch.from_numpy(o).to(torch.bfloat16)
    for out, lse in outs:
        assert torch.equal(out.cpu(), ref_o) and np.array_equal(lse.cpu().numpy(), l)


def test_persistent_launches_on_two_streams():
    B, Hq, Hkv, T, D = 8, 16, 4, 2112, 128
    q1, k1, v1 = (t.cuda() for t in inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=41))
    q2, k2, v2 = (t.cuda() for t in inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=42))
    want1 = binding.attn_fwd(q1, k1, v1)
    want2 = binding.attn_fwd(q2, k2, v2)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    got = []
    for _ in range(3):
        o1, l1 = torch.empty_like(q1), torch.empty_like(want1[1])
        o2, l2 = torch.empty_like(q2), torch.empty_like(want2[1])
        binding.attn_fwd_into(q1, k1, v1, o1, l1, True, None, stream=s1)
        binding.attn_fwd_into(q2, k2, v2, o2, l2, True, None, stream=s2)
        got.append((o1, l1, o2, l2))
    torch.cuda.synchronize()
    for o1, l1, o2, l2 in got:
        assert torch.equal(o1, want1[0]) and torch.equal(l1, want1[1])
        assert torch.equal(o2, want2[0]) and torch.equal(l2, want2[1])


# Every tile configuration the table may pick from (tessera_attn_fwd_with_config),
# for each head size, causal or not, with T ragged and a multiple of the key
# tile: 1056 work items at four heads per workgroup, so the persistent ones do
# run persistently.  Sampled rows of each output against the oracle.
_CONFIG_INPUTS = {}


def _config_case(D, T):
    if (D, T) not in _CONFIG_INPUTS:
        q, k, v = inputs.make_qkv(8, 16, 4, T, D, "bf16", seed=D + T)
        rows = np.unique(np.random.default_rng(D + T).integers(0, 8 * 16 * T, 160)).astype(np.int64)
        bits = [inputs.bits(t) for t in (q, k, v)]
        refs = {c: oracle.attn_rows(*bits, c, inputs.default_scale(D), rows) for c in (True, False)}
        _CONFIG_INPUTS[(D, T)] = ([t.cuda() for t in (q, k, v)], rows, refs)
    return _CONFIG_INPUTS[(D, T)]


def _all_configs(D, T):
    from attention_flashattention_fwd_amd import autotune
    return autotune.configs(4, T, D)


@pytest.mark.parametrize("D,T,causal,cfg", [
    (D, T, causal, cfg) for D in (128, 64, 32) for T in (2112, 2100) for causal in (True, False)
    for cfg in _all_configs(D, T)])
def test_every_tile_configuration(D, T, causal, cfg):
    (q, k, v), rows, refs = _config_case(D, T)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    binding.attn_fwd_with_config_into(q, k, v, out, lse, binding.TileConfig(*cfg), causal)
    torch.cuda.synchronize()
    idx = torch.from_numpy(rows).to(q.device)
    o = out.reshape(-1, D)[idx].float().cpu().numpy().astype(np.float64)
    l = lse.reshape(-1)[idx].cpu().numpy().astype(np.float64)
    check_close(o, l, *refs[causal], "bf16", f"D={D} T={T} causal={causal} config={cfg}")


# Two workgroups per CU take the second round of each XCD's workgroups in
# reverse.  These grids give the XCDs between one and two rounds (32 and 64
# workgroups on 32 CUs), uneven across the XCDs when the item count is not a
# multiple of 8, so the reversed round is partial; every element is compared.
@pytest.mark.parametrize("B,T,causal", [(6, 2048, True), (5, 1984, True), (5, 1984, False),
                                        (3, 4032, True)])
def test_paired_launch_with_a_partial_second_round(B, T, causal):
    Hq, Hkv, D = 8, 2, 64
    items = (T // 64) * B * Hkv
    assert 8 * 32 < items < 8 * 64, items
    q, k, v = inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=B + T)
    scale = inputs.default_scale(D)
    say(f"case paired partial round B={B} T={T} causal={causal} items={items}")
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out = torch.empty_like(qd)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
    binding.attn_fwd_with_config_into(qd, kd, vd, out, lse, binding.TileConfig(4, 32, 2, 0),
                                      causal)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    O_ref, l_ref = oracle.attn_fwd(inputs.bits(q), inputs.bits(k), inputs.bits(v), causal, scale)
    check_close(o, l, O_ref, l_ref, "bf16", f"paired B={B} T={T} causal={causal}")


def test_tile_configurations_the_sizes_do_not_allow():
    q, k, v = (t.cuda() for t in inputs.make_qkv(1, 12, 4, 100, 128, "bf16", seed=1))
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[:3], dtype=torch.float32, device=q.device)
    for cfg in [(2, 32, 1, 0),    # 2 does not divide the group of 3
                (1, 64, 1, 0),    # 64 rows per wave at D = 128
                (1, 32, 2, 0),    # two workgroups per CU at D = 128
                (3, 32, 1, 0), (1, 48, 1, 0), (1, 32, 3, 0), (1, 32, 1, 2)]:
        with pytest.raises(RuntimeError, match="unsupported"):
            binding.attn_fwd_with_config_into(q, k, v, out, lse, binding.TileConfig(*cfg))
    q64, k64, v64 = (t.cuda() for t in inputs.make_qkv(1, 4, 4, 100, 64, "bf16", seed=1))
    with pytest.raises(RuntimeError, match="unsupported"):   # ragged T, two per CU
        binding.attn_fwd_with_config_into(q64, k64, v64, torch.empty_like(q64),
                                          torch.empty(q64.shape[:3], device=q64.device),
                                          binding.TileConfig(1, 32, 2, 0))


# (D, rate, seed, B, Hq, Hkv, T, causal): the last two run the two-workgroups-
# per-CU build (2048 workgroups) and the two-query-blocks-per-wave build.
GROWING = [
    (64, 8.0, 5, 1, 8, 2, 512, True),
    (128, 8.0, 5, 1, 8, 2, 512, True),
    (128, 10.0, 7, 1, 8, 2, 512, True),
    (32, 10.0, 7, 1, 8, 2, 512, True),
    (64, 2.0, 9, 128, 32, 8, 128, True),
    (64, 8.0, 5, 1, 8, 2, 512, False),
]


@pytest.mark.parametrize("D,rate,seed,B,Hq,Hkv,T,causal", GROWING)
def test_scores_growing_along_the_keys(D, rate, seed, B, Hq, Hkv, T, causal):
    """Key rows grow with position, so later tiles beat the running max by far
    more than the lazy-rescale bound: the rescale path runs mid-sequence.  The
    late rows attend almost entirely to one key, which is where a row sum of
    unrounded p against a P V product of rounded p would show."""
    q, k, v = inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=seed)
    grow = (1.0 + torch.arange(T, dtype=torch.float32) / rate).view(1, 1, T, 1)
    k = (k.float() * grow).to(torch.bfloat16)
    scale = inputs.default_scale(D)
    say(f"case growing keys B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} rate={rate} seed={seed} "
        f"causal={causal}")
    o, l = run_gpu(q, k, v, causal, scale)
    O_ref, l_ref = oracle.attn_fwd(inputs.bits(q), inputs.bits(k), inputs.bits(v), causal, scale)
    check_close(o, l, O_ref, l_ref, "bf16")
    assert l_ref.max() - l_ref.min() > 64 * math.log(2)   # the spread that forces rescales


def test_offsets_past_int32():
    """Q and O of 8200 x 32 x 128 x 64 elements (more than 2^31): the last
    eight batch elements start past 2^31 elements, where any 32-bit element
    or byte offset would wrap.  Those and batch element 0 are compared whole
    against the oracle."""
    B, Hq, Hkv, T, D = 8200, 32, 8, 128, 64
    assert B * Hq * T * D > 2 ** 31 and 8192 * Hq * T * D == 2 ** 31
    dev = torch.device("cuda:0")
    say(f"case int32-overflowing offsets B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} causal")
    q, k, v = inputs.make_qkv_on_device(B, Hq, Hkv, T, D, seed=21, device=dev)
    scale = inputs.default_scale(D)
    out, lse = binding.attn_fwd(q, k, v, causal=True, scale=scale)
    torch.cuda.synchronize()
    for b in (0, 8192, 8195, B - 1):
        qs, ks, vs = (t[b:b + 1].cpu() for t in (q, k, v))
        O_ref, l_ref = oracle.attn_fwd(inputs.bits(qs), inputs.bits(ks), inputs.bits(vs), True,
                                       scale)
        o = out[b:b + 1].float().cpu().numpy().astype(np.float64)
        l = lse[b:b + 1].cpu().numpy().astype(np.float64)
        check_close(o, l, O_ref, l_ref, "bf16", f"batch element {b}")
    del q, k, v, out, lse
    torch.cuda.empty_cache()


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("D,causal", [(32, True), (64, False), (128, True)])
def test_identical_value_rows(dtype, D, causal):
    """With every V row of a head equal, each output row is that row: the
    softmax weights sum to one (for bf16 exactly the rounded weights the P V
    product uses, so O comes back bit for bit)."""
    B, Hq, Hkv, T = 2, 8, 2, 333
    q, k, v = inputs.make_qkv(B, Hq, Hkv, T, D, dtype, seed=D + 1)
    v = v[:, :, :1, :].expand(B, Hkv, T, D).contiguous()
    say(f"case identical V rows B={B} Hq={Hq} Hkv={Hkv} T={T} D={D} {dtype} causal={causal}")
    o, _ = run_gpu(q, k, v, causal, inputs.default_scale(D))
    want = np.repeat(v[:, :, :1, :].float().numpy().astype(np.float64), Hq // Hkv, axis=1)
    err = np.abs(o - want).max()
    say(f"max |O - v0| {err:.3e}")
    assert err == 0.0 if dtype == "bf16" else err <= F32_MAX


@pytest.mark.parametrize("B,Hq,Hkv,T,D,causal", [
    (1, 2, 1, 1, 32, True), (2, 4, 2, 65, 64, True), (1, 4, 4, 130, 128, False),
    (1, 8, 2, 300, 128, True), (2, 2, 2, 77, 32, False)])
def test_edge_shapes_fp32(B, Hq, Hkv, T, D, causal):
    full_case(B, Hq, Hkv, T, D, "fp32", causal, seed=T)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("scale", [-0.125, 0.0, 0.5, 1e-3])
def test_scale_values(dtype, scale):
    full_case(2, 8, 2, 150, 64, dtype, True, scale=scale, seed=7)


# Large scales make every row sharply peaked and the running max rise many
# times along a row (a raise needs a score about 33 / (scale log2 e) above the
# max so far), which exercises the rescaling path of every build: the default
# pick and two workgroups per CU (D = 64, whole key tiles).
@pytest.mark.parametrize("scale", [8.0, -8.0, 30.0])
@pytest.mark.parametrize("cfg", [None, (4, 32, 2, 0)])
def test_large_scales(scale, cfg):
    B, Hq, Hkv, T, D = 2, 8, 2, 1024, 64
    q, k, v = inputs.make_qkv(B, Hq, Hkv, T, D, "bf16", seed=11)
    say(f"case large scale={scale} config={cfg}")
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    if cfg is None:
        out, lse = binding.attn_fwd(qd, kd, vd, causal=True, scale=scale)
    else:
        out = torch.empty_like(qd)
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
        binding.attn_fwd_with_config_into(qd, kd, vd, out, lse, binding.TileConfig(*cfg), True,
                                          scale)
    torch.cuda.synchronize()
    o = out.float().cpu().numpy().astype(np.float64)
    l = lse.cpu().numpy().astype(np.float64)
    O_ref, l_ref = oracle.attn_fwd(inputs.bits(q), inputs.bits(k), inputs.bits(v), True, scale)
    check_close(o, l, O_ref, l_ref, "bf16", f"scale={scale} config={cfg}")


@pytest.mark.parametrize("mode", ["elements", "rows"])
def test_outliers_small(mode):
    full_case(2, 8, 2, 600, 64, "bf16", True, seed=3, outliers=mode)


def test_side_stream_and_repeatability():
    q, k, v = (t.cuda() for t in inputs.make_qkv(2, 8, 2, 300, 64, "bf16", seed=11))
    out1, lse1 = binding.attn_fwd(q, k, v)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        out2 = torch.empty_like(q)
        lse2 = torch.empty_like(lse1)
        binding.attn_fwd_into(q, k, v, out2, lse2, True, None, stream=s)
    s.synchronize()
    torch.cuda.synchronize()
    assert torch.equal(out1, out2) and torch.equal(lse1, lse2)


def test_binding_argument_checks():
    q = torch.zeros(1, 4, 16, 64, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 16, 64, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        binding.attn_fwd(q, k.float(), k)
    with pytest.raises(ValueError):
        binding.attn_fwd(q.transpose(1, 2), k, k)
    with pytest.raises(RuntimeError, match="shape"):
        binding.attn_fwd(torch.zeros(1, 3, 16, 64, dtype=torch.bfloat16, device="cuda"), k, k)
    with pytest.raises(RuntimeError, match="D must be 32, 64 or 128"):
        binding.attn_fwd(q[..., :48].contiguous(), k[..., :48].contiguous(),
                         k[..., :48].contiguous())


# -- the full-size workloads, in the launch configuration the bench times ----
def gpu_workload(w):
    q, k, v = inputs.make_workload(w)
    dev = torch.device("cuda:0")
    qd, kd, vd = (t.to(dev) for t in (q, k, v))
    out, lse = binding.attn_fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
    torch.cuda.synchronize()
    # every row: finite, and (causal) row 0 equals V[0] exactly
    assert torch.isfinite(out.float()).all() and torch.isfinite(lse).all()
    G = w.Hq // w.Hkv
    if w.causal:
        assert torch.equal(out[:, :, 0], vd[:, :, 0].repeat_interleave(G, dim=1))
        s0 = (qd[:, :, 0].float() * kd[:, :, 0].float().repeat_interleave(G, dim=1)).sum(-1)
        assert torch.allclose(lse[:, :, 0], s0 * w.scale, atol=1e-3, rtol=0)
    return q, k, v, out, lse


@pytest.mark.parametrize("name", ["t2048", "t2048_full", "t4096_outliers",
                                  "t4096_outlier_rows"])
def test_full_size_workload_every_element(name):
    """T=2048 (causal and not) and T=4096 (both outlier readings) at full size:
    every element of out and lse against the oracle."""
    w = inputs.WORKLOADS[name]
    say(f"workload {name}: {w.describe()}, every element")
    q, k, v, out, lse = gpu_workload(w)
    O_ref, l_ref = oracle.attn_fwd(inputs.bits(q), inputs.bits(k), inputs.bits(v), w.causal,
                                   w.scale)
    check_close(out.float().cpu().numpy().astype(np.float64),
                lse.cpu().numpy().astype(np.float64), O_ref, l_ref, w.dtype, name)


def test_full_size_long_context_whole_groups():
    """The long-context workload (B=1 Hq=32 Hkv=8 T=16384 D=128) at full size:
    every element of out and lse of two whole GQA groups, KV heads 0 and 7
    with their query heads 0-3 and 28-31, against the oracle; the other
    groups are checked on 400 random rows."""
    w = inputs.WORKLOADS["t16384_d128"]
    say(f"workload {w.name}: {w.describe()}, KV heads 0 and 7 whole")
    q, k, v, out, lse = gpu_workload(w)
    G = w.Hq // w.Hkv
    for g in (0, w.Hkv - 1):
        hs = slice(g * G, (g + 1) * G)
        O_ref, l_ref = oracle.attn_fwd(inputs.bits(q[:, hs]), inputs.bits(k[:, g:g + 1]),
                                       inputs.bits(v[:, g:g + 1]), w.causal, w.scale)
        check_close(out[:, hs].float().cpu().numpy().astype(np.float64),
                    lse[:, hs].cpu().numpy().astype(np.float64), O_ref, l_ref, w.dtype,
                    f"KV head {g}")
    rows = np.unique(np.random.default_rng(5).integers(0, w.B * w.Hq * w.T, 400)).astype(np.int64)
    O_ref, l_ref = oracle.attn_rows(inputs.bits(q), inputs.bits(k), inputs.bits(v), w.causal,
                                    w.scale, rows)
    idx = torch.from_numpy(rows).to(out.device)
    o = out.reshape(-1, w.D)[idx].float().cpu().numpy().astype(np.float64)
    l = lse.reshape(-1)[idx].cpu().numpy().astype(np.float64)
    check_close(o, l, O_ref, l_ref, w.dtype, "random rows")
