"""Pins of the fp64 attention oracle to facts other than itself.

Each `pin_*` function takes a loaded oracle library and raises AssertionError
when the oracle breaks the fact it checks.  `test_oracle.py` runs every pin on
the real oracle, and also on deliberately broken copies of it, each of which
at least one pin must reject.

What fixes each fact:
  * hand-worked example (tests/golden): values derived by hand from the
    softmax-attention definition;
  * mpmath at 50 digits: brute force on tiny inputs;
  * torch's scaled_dot_product_attention in float64 on the CPU: an
    independent library routine, with K/V heads repeated for GQA;
  * closed forms and invariants of softmax attention: uniform weights when
    all scores are equal, row 0 under the causal mask, identical value rows,
    identity values exposing the weights, GQA equal to repeated-head MHA,
    key shift and key permutation invariance.
"""
from __future__ import annotations

import math
from fractions import Fraction
from pathlib import Path

import mpmath
import numpy as np
import torch

GOLDEN = Path(__file__).resolve().parent / "golden"


# ---------------------------------------------------------------------------
# input helpers (plain numpy draws; no attention arithmetic)
# ---------------------------------------------------------------------------
def rand_inputs(B, Hq, Hkv, T, D, dtype, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, T, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, T, D)).astype(np.float32)
    return tuple(as_dtype(a, dtype) for a in (q, k, v))


def as_dtype(a, dtype):
    """float32 array -> the oracle's input form for `dtype` (bf16: RNE bits)."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    if dtype == "fp32":
        return a
    t = torch.from_numpy(a).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def values(a):
    """Exact float64 values of an oracle input array."""
    if a.dtype == np.float32:
        return a.astype(np.float64)
    return (a.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp32(x):
    return float(np.float32(x))


# ---------------------------------------------------------------------------
# the hand-worked golden example
# ---------------------------------------------------------------------------
def _parse_value(tok):
    if tok.startswith("ln(") and tok.endswith(")"):
        return math.log(int(tok[3:-1]))
    return float(Fraction(tok))


def load_golden(name="hand_worked_gqa_t4.txt"):
    arrays = {}
    shape = scale = None
    for raw in (GOLDEN / name).read_text().splitlines():
        line = raw.strip()
        if not line or line.startswith("#"):
            continue
        key, vals = line.split(":", 1)
        parts = key.split()
        toks = vals.split()
        if parts[0] == "shape":
            shape = tuple(int(t) for t in toks)
            B, Hq, Hkv, T, D = shape
            for nm, shp in (("q", (B, Hq, T, D)), ("k", (B, Hkv, T, D)), ("v", (B, Hkv, T, D)),
                            ("causal_O", (B, Hq, T, D)), ("full_O", (B, Hq, T, D)),
                            ("causal_lse", (B, Hq, T)), ("full_lse", (B, Hq, T))):
                arrays[nm] = np.full(shp, np.nan)
            continue
        if parts[0] == "scale":
            assert toks == ["fp32_ln2"]
            scale = fp32(math.log(2.0))
            continue
        idx = tuple(int(t) for t in parts[1:])
        arrays[parts[0]][idx] = [_parse_value(t) for t in toks]
    for nm, a in arrays.items():
        assert not np.isnan(a).any(), f"golden array {nm} incomplete"
    return shape, scale, arrays


def pin_golden(lib):
    shape, scale, g = load_golden()
    for dtype in ("fp32", "bf16"):
        q, k, v = (as_dtype(g[n], dtype) for n in ("q", "k", "v"))
        for mode, causal in (("causal", True), ("full", False)):
            O, lse = lib.attn_fwd(q, k, v, causal, scale)
            assert np.abs(O - g[f"{mode}_O"]).max() < 5e-8, (dtype, mode, O)
            assert np.abs(lse - g[f"{mode}_lse"]).max() < 5e-8, (dtype, mode, lse)


# ---------------------------------------------------------------------------
# brute force in 50-digit arithmetic on tiny inputs
# ---------------------------------------------------------------------------
def mp_attention(qv, kv, vv, causal, scale):
    """Softmax attention by brute force with mpmath (no max subtraction).  With
    Tq query rows and Tk key rows, query row i is at sequence position
    i + Tk - Tq and, under the causal mask, sees keys 0 .. i + Tk - Tq."""
    mpmath.mp.dps = 50
    B, Hq, T, D = qv.shape
    Hkv, Tk = kv.shape[1], kv.shape[2]
    G = Hq // Hkv
    O = np.zeros((B, Hq, T, D))
    lse = np.zeros((B, Hq, T))
    sc = mpmath.mpf(scale)
    for b in range(B):
        for h in range(Hq):
            kvh = h // G
            for i in range(T):
                keys = range(i + (Tk - T) + 1) if causal else range(Tk)
                e = []
                for j in keys:
                    dot = mpmath.fsum(mpmath.mpf(qv[b, h, i, d]) * mpmath.mpf(kv[b, kvh, j, d])
                                      for d in range(D))
                    e.append(mpmath.exp(sc * dot))
                Z = mpmath.fsum(e)
                for d in range(D):
                    num = mpmath.fsum(e[n] * mpmath.mpf(vv[b, kvh, j, d])
                                      for n, j in enumerate(keys))
                    O[b, h, i, d] = float(num / Z)
                lse[b, h, i] = float(mpmath.log(Z))
    return O, lse


def pin_mpmath(lib):
    cases = [(1, 1, 1, 1, 1), (1, 2, 1, 5, 3), (2, 4, 2, 8, 4), (1, 3, 3, 6, 2), (2, 4, 1, 7, 4)]
    for n, (B, Hq, Hkv, T, D) in enumerate(cases):
        for dtype in ("fp32", "bf16"):
            q, k, v = rand_inputs(B, Hq, Hkv, T, D, dtype, seed=100 + n)
            scale = fp32(0.7 + 0.1 * n)
            for causal in (True, False):
                O, lse = lib.attn_fwd(q, k, v, causal, scale)
                Om, lm = mp_attention(values(q), values(k), values(v), causal, scale)
                assert np.abs(O - Om).max() <= 1e-12, (B, Hq, Hkv, T, D, dtype, causal)
                assert np.abs(lse - lm).max() <= 1e-12, (B, Hq, Hkv, T, D, dtype, causal)


# ---------------------------------------------------------------------------
# a library routine: torch SDPA in float64 on the CPU
# ---------------------------------------------------------------------------
def pin_torch_sdpa(lib):
    cases = [(2, 6, 2, 37, 16, True), (2, 6, 2, 37, 16, False), (1, 4, 4, 64, 32, True),
             (3, 8, 1, 19, 8, True)]
    for n, (B, Hq, Hkv, T, D, causal) in enumerate(cases):
        for dtype in ("fp32", "bf16"):
            q, k, v = rand_inputs(B, Hq, Hkv, T, D, dtype, seed=200 + n)
            scale = fp32(1.0 / math.sqrt(D))
            O, lse = lib.attn_fwd(q, k, v, causal, scale)
            qt, kt, vt = (torch.from_numpy(values(a)) for a in (q, k, v))
            G = Hq // Hkv
            kt = kt.repeat_interleave(G, dim=1)
            vt = vt.repeat_interleave(G, dim=1)
            ref = torch.nn.functional.scaled_dot_product_attention(
                qt, kt, vt, is_causal=causal, scale=scale)
            assert np.abs(O - ref.numpy()).max() <= 1e-12, (B, Hq, Hkv, T, D, causal, dtype)
            s = (qt @ kt.transpose(-1, -2)) * scale
            if causal:
                s = s.masked_fill(torch.ones(T, T, dtype=torch.bool).triu(1), float("-inf"))
            assert np.abs(lse - torch.logsumexp(s, dim=-1).numpy()).max() <= 1e-12


# ---------------------------------------------------------------------------
# closed forms and invariants
# ---------------------------------------------------------------------------
def pin_weights_sum_to_one(lib):
    """V = identity (T <= D): O's row i is the weight row of query i."""
    B, Hq, Hkv, T, D = 2, 4, 2, 12, 16
    q, k, _ = rand_inputs(B, Hq, Hkv, T, D, "fp32", seed=3)
    eye = np.zeros((B, Hkv, T, D), np.float32)
    for j in range(T):
        eye[:, :, j, j] = 1.0
    for causal in (True, False):
        O, _ = lib.attn_fwd(q, k, eye, causal, 0.5)
        W = O[..., :T]
        assert np.abs(W.sum(-1) - 1.0).max() <= 1e-13
        assert (W >= 0).all() and np.abs(O[..., T:]).max() == 0.0
        if causal:
            assert np.abs(np.triu(W, 1)).max() == 0.0, "a future key got weight"
        else:
            assert W.min() > 0.0


def pin_probs_export(lib):
    q, k, v = rand_inputs(1, 2, 1, 9, 4, "bf16", seed=4)
    for causal in (True, False):
        O, lse, P = lib.attn_probs(q, k, v, causal, 0.6)
        O2, lse2 = lib.attn_fwd(q, k, v, causal, 0.6)
        assert np.array_equal(O, O2) and np.array_equal(lse, lse2)
        assert np.abs(P.sum(-1) - 1.0).max() <= 1e-13
        Vrep = np.repeat(values(v), 2, axis=1)
        assert np.abs(P @ Vrep - O).max() <= 1e-13
        if causal:
            assert np.abs(np.triu(P, 1)).max() == 0.0


def pin_causal_row0(lib):
    """Query 0 sees only key 0: O = V[0] exactly, lse = scale*q0.k0."""
    B, Hq, Hkv, T, D = 2, 4, 2, 10, 8
    for dtype in ("fp32", "bf16"):
        q, k, v = rand_inputs(B, Hq, Hkv, T, D, dtype, seed=5)
        O, lse = lib.attn_fwd(q, k, v, True, 0.3)
        qv, kv, vv = values(q), values(k), values(v)
        for b in range(B):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                assert np.array_equal(O[b, h, 0], vv[b, g, 0])
                dot = math.fsum(qv[b, h, 0] * kv[b, g, 0])
                assert abs(lse[b, h, 0] - 0.3 * dot) <= 1e-12


def pin_identical_value_rows(lib):
    B, Hq, Hkv, T, D = 1, 4, 2, 15, 8
    q, k, _ = rand_inputs(B, Hq, Hkv, T, D, "fp32", seed=6)
    c = np.arange(1, D + 1, dtype=np.float32) * np.float32(0.25)
    v = np.broadcast_to(c, (B, Hkv, T, D)).copy()
    for causal in (True, False):
        O, _ = lib.attn_fwd(q, k, v, causal, 0.9)
        assert np.abs(O - c.astype(np.float64)).max() <= 1e-12


def pin_uniform_scores(lib):
    """All scores equal (Q = 0, or scale = 0): O_i = mean of visible V rows,
    lse_i = ln(#visible keys)."""
    B, Hq, Hkv, T, D = 1, 2, 1, 11, 4
    q, k, v = rand_inputs(B, Hq, Hkv, T, D, "fp32", seed=7)
    vv = values(v)
    for qq, scale in ((np.zeros_like(q), 0.5), (q, 0.0)):
        O, lse = lib.attn_fwd(qq, k, v, True, scale)
        for i in range(T):
            assert np.abs(O[0, :, i] - vv[0, 0, : i + 1].mean(0)).max() <= 1e-13
            assert np.abs(lse[0, :, i] - math.log(i + 1)).max() <= 1e-13
        O, lse = lib.attn_fwd(qq, k, v, False, scale)
        assert np.abs(O[0, :, :] - vv[0, 0].mean(0)).max() <= 1e-13
        assert np.abs(lse - math.log(T)).max() <= 1e-13


def pin_gqa_equals_repeated_mha(lib):
    B, Hq, Hkv, T, D = 2, 8, 2, 13, 8
    for dtype in ("fp32", "bf16"):
        q, k, v = rand_inputs(B, Hq, Hkv, T, D, dtype, seed=8)
        G = Hq // Hkv
        kr = np.ascontiguousarray(np.repeat(k, G, axis=1))
        vr = np.ascontiguousarray(np.repeat(v, G, axis=1))
        for causal in (True, False):
            O, lse = lib.attn_fwd(q, k, v, causal, 0.4)
            O2, lse2 = lib.attn_fwd(q, kr, vr, causal, 0.4)
            assert np.array_equal(O, O2) and np.array_equal(lse, lse2)
        # and the repeat is not a no-op: a different head map changes the result
        O3, _ = lib.attn_fwd(q, np.ascontiguousarray(np.tile(k, (1, G, 1, 1))),
                             np.ascontiguousarray(np.tile(v, (1, G, 1, 1))), True, 0.4)
        assert not np.allclose(O3, O)


def pin_lse_closed_form(lib):
    B, Hq, Hkv, T, D = 1, 3, 1, 17, 8
    q, k, v = rand_inputs(B, Hq, Hkv, T, D, "fp32", seed=9)
    qv, kv = values(q), values(k)
    for causal in (True, False):
        _, lse = lib.attn_fwd(q, k, v, causal, 0.35)
        for h in range(Hq):
            for i in range(T):
                n = i + 1 if causal else T
                sc = [0.35 * math.fsum(qv[0, h, i] * kv[0, 0, j]) for j in range(n)]
                assert abs(lse[0, h, i] - np.logaddexp.reduce(np.array(sc))) <= 1e-12


def pin_key_shift(lib):
    """k_j -> k_j + c leaves O unchanged and moves lse_i by scale*q_i.c."""
    B, Hq, Hkv, T, D = 1, 2, 1, 20, 8
    q, k, v = rand_inputs(B, Hq, Hkv, T, D, "fp32", seed=10)
    k = (np.round(k * 1024.0) / 1024.0).astype(np.float32)  # so that k + c is exact in fp32
    c = np.float32(40.0) * np.sign(values(q)[0, 0, 0]).astype(np.float32)
    k2 = (k + c).astype(np.float32)
    shift_ok = np.array_equal(values(k2) - values(k), np.broadcast_to(c.astype(np.float64),
                                                                      k.shape))
    assert shift_ok, "shift must be exact in fp32 for this pin"
    for causal in (True, False):
        O, lse = lib.attn_fwd(q, k, v, causal, 0.25)
        O2, lse2 = lib.attn_fwd(q, k2, v, causal, 0.25)
        assert np.abs(O2 - O).max() <= 1e-11
        delta = 0.25 * (values(q) @ c.astype(np.float64))
        assert np.abs(lse2 - lse - delta).max() <= 1e-10


def pin_key_permutation(lib):
    B, Hq, Hkv, T, D = 2, 4, 2, 16, 8
    q, k, v = rand_inputs(B, Hq, Hkv, T, D, "bf16", seed=11)
    perm = np.random.default_rng(12).permutation(T)
    kp = np.ascontiguousarray(k[:, :, perm])
    vp = np.ascontiguousarray(v[:, :, perm])
    O, lse = lib.attn_fwd(q, k, v, False, 0.2)
    O2, lse2 = lib.attn_fwd(q, kp, vp, False, 0.2)
    assert np.abs(O2 - O).max() <= 1e-13 and np.abs(lse2 - lse).max() <= 1e-13
    # with the causal mask the order matters
    O3, _ = lib.attn_fwd(q, kp, vp, True, 0.2)
    O4, _ = lib.attn_fwd(q, k, v, True, 0.2)
    assert not np.allclose(O3, O4)


# ---------------------------------------------------------------------------
# continuation of a cached sequence: Tq query rows against Tk key rows
# ---------------------------------------------------------------------------
def rand_kv_inputs(B, Hq, Hkv, Tq, Tk, D, dtype, seed):
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, Hq, Tq, D)).astype(np.float32)
    k = rng.standard_normal((B, Hkv, Tk, D)).astype(np.float32)
    v = rng.standard_normal((B, Hkv, Tk, D)).astype(np.float32)
    return tuple(as_dtype(a, dtype) for a in (q, k, v))


def pin_kv_mpmath(lib):
    """Brute force at 50 digits with the causal mask aligned to the last key."""
    cases = [(1, 2, 1, 1, 5, 3, True), (2, 4, 2, 3, 8, 4, True), (1, 3, 3, 6, 6, 2, True),
             (2, 4, 1, 2, 7, 4, False), (1, 2, 1, 5, 3, 2, False)]
    for n, (B, Hq, Hkv, Tq, Tk, D, causal) in enumerate(cases):
        for dtype in ("fp32", "bf16"):
            q, k, v = rand_kv_inputs(B, Hq, Hkv, Tq, Tk, D, dtype, seed=400 + n)
            scale = fp32(0.6 + 0.1 * n)
            O, lse = lib.attn_fwd_kv(q, k, v, causal, scale)
            Om, lm = mp_attention(values(q), values(k), values(v), causal, scale)
            assert np.abs(O - Om).max() <= 1e-12, (B, Hq, Hkv, Tq, Tk, D, dtype, causal)
            assert np.abs(lse - lm).max() <= 1e-12, (B, Hq, Hkv, Tq, Tk, D, dtype, causal)


def pin_kv_suffix_of_full_forward(lib):
    """The pages' serving invariant: the last Tq rows of a full forward over T
    positions equal Tq new rows computed against the cached T keys."""
    B, Hq, Hkv, T, D = 2, 4, 2, 29, 8
    q, k, v = rand_inputs(B, Hq, Hkv, T, D, "bf16", seed=17)
    for causal in (True, False):
        O, lse = lib.attn_fwd(q, k, v, causal, 0.3)
        for Tq in (1, 2, 13, T):
            Ok, lk = lib.attn_fwd_kv(np.ascontiguousarray(q[:, :, T - Tq:]), k, v, causal, 0.3)
            assert np.array_equal(Ok, O[:, :, T - Tq:]), (causal, Tq)
            assert np.array_equal(lk, lse[:, :, T - Tq:]), (causal, Tq)


def pin_kv_torch_sdpa(lib):
    """torch SDPA in float64 with an explicit mask: key j visible to query row
    i iff j <= i + Tk - Tq."""
    for n, (B, Hq, Hkv, Tq, Tk, D) in enumerate([(2, 6, 2, 9, 40, 16), (1, 4, 4, 33, 33, 8),
                                                (1, 8, 1, 1, 70, 32)]):
        q, k, v = rand_kv_inputs(B, Hq, Hkv, Tq, Tk, D, "bf16", seed=500 + n)
        scale = fp32(1.0 / math.sqrt(D))
        qt, kt, vt = (torch.from_numpy(values(a)) for a in (q, k, v))
        kt = kt.repeat_interleave(Hq // Hkv, dim=1)
        vt = vt.repeat_interleave(Hq // Hkv, dim=1)
        visible = torch.arange(Tk)[None, :] <= torch.arange(Tq)[:, None] + (Tk - Tq)
        O, lse = lib.attn_fwd_kv(q, k, v, True, scale)
        ref = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, attn_mask=visible,
                                                               scale=scale)
        assert np.abs(O - ref.numpy()).max() <= 1e-12, (B, Hq, Hkv, Tq, Tk, D)
        s = ((qt @ kt.transpose(-1, -2)) * scale).masked_fill(~visible, float("-inf"))
        assert np.abs(lse - torch.logsumexp(s, dim=-1).numpy()).max() <= 1e-12


def pin_rows_entry(lib):
    """The sampled-rows entry returns exactly the rows of the full call."""
    B, Hq, Hkv, T, D = 2, 4, 2, 33, 16
    q, k, v = rand_inputs(B, Hq, Hkv, T, D, "bf16", seed=13)
    rows = np.array([0, 1, 32, 33, 70, B * Hq * T - 1], np.int64)
    for causal in (True, False):
        O, lse = lib.attn_fwd(q, k, v, causal, 0.125)
        Or, lr = lib.attn_rows(q, k, v, causal, 0.125, rows)
        assert np.array_equal(Or, O.reshape(-1, D)[rows])
        assert np.array_equal(lr, lse.reshape(-1)[rows])


ALL_PINS = [pin_golden, pin_mpmath, pin_torch_sdpa, pin_weights_sum_to_one, pin_probs_export,
            pin_causal_row0, pin_identical_value_rows, pin_uniform_scores,
            pin_gqa_equals_repeated_mha, pin_lse_closed_form, pin_key_shift,
            pin_key_permutation, pin_rows_entry, pin_kv_mpmath, pin_kv_suffix_of_full_forward,
            pin_kv_torch_sdpa]
