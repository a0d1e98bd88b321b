"""CPU tests of the fp64 oracle: its pins, planted mistakes, and its argument checks."""
from __future__ import annotations

import ctypes
import subprocess
from pathlib import Path

import numpy as np
import pytest

import oracle
from oracle.oracle import BWD_SOURCE, PAGED_SOURCE, RMS_SOURCE, SOURCE, OracleLib
from tests import oracle_pins
from tests.oracle_pins import ALL_PINS, rand_inputs
from tests.attn_bwd_pins import ALL_BWD_PINS
from tests.paged_pins import ALL_PAGED_PINS
from tests.rmsnorm_pins import ALL_RMS_PINS


@pytest.fixture(scope="module")
def lib():
    return oracle.load()


@pytest.mark.parametrize("pin", ALL_PINS + ALL_RMS_PINS + ALL_BWD_PINS + ALL_PAGED_PINS,
                         ids=lambda f: f.__name__)
def test_pin(lib, pin):
    pin(lib)


# Plausible mistakes, each planted in a copy of the oracle source.  Every one
# must make at least one pin fail; a mutant that passes them all would mean the
# pins leave that part of the oracle unchecked.
MUTANTS = {
    "interleaved_head_map": ("const int g = h / G;", "const int g = h % Hkv;"),
    "mask_hides_diagonal": ("causal ? pos + 1 : Tk", "causal ? pos : Tk"),
    "mask_leaks_next_key": ("causal ? pos + 1 : Tk", "causal ? (pos + 2 < Tk ? pos + 2 : Tk) : Tk"),
    "mask_ignored": ("causal ? pos + 1 : Tk", "Tk"),
    "cache_offset_dropped": ("const int pos = i + (Tk - Tq);", "const int pos = i;"),
    "cache_offset_reversed": ("const int pos = i + (Tk - Tq);", "const int pos = i + (Tq - Tk);"),
    "key_stride_from_queries": ("* Tk * D;", "* Tq * D;"),
    "query_stride_from_keys": ("* Tq + i) * D;", "* Tk + i) * D;"),
    "scale_dropped": ("s[j] = scale * dot;", "s[j] = dot;"),
    "scale_squared": ("s[j] = scale * dot;", "s[j] = scale * scale * dot;"),
    "lse_without_max": ("*lse = m + log(Z);", "*lse = log(Z);"),
    "lse_log2": ("*lse = m + log(Z);", "*lse = m + log2(Z);"),
    "unnormalised": ("const double w = p[j] / Z;", "const double w = p[j];"),
    "scores_use_v": ("dot += widen(q, dtype, qrow + d) * widen(k,",
                     "dot += widen(q, dtype, qrow + d) * widen(v,"),
    "exp_sign_flipped": ("p[j] = exp(s[j] - m);", "p[j] = exp(m - s[j]);"),
    "dropped_last_dim": ("for (int d = 0; d < D; ++d)\n            dot +=",
                         "for (int d = 0; d < D - 1; ++d)\n            dot +="),
    "bf16_widen_shift": ("<< 16;", "<< 15;"),
    "query_row_stride": ("* Tq + i) * D;", "* Tq + i) * D + (i > 0);"),
    "value_from_query_head": ("o[d] += w * widen(v, dtype, kv0 +",
                              "o[d] += w * widen(v, dtype, (int64_t)0 * kv0 +"),
}


# The same for the RMSNorm oracle.
RMS_MUTANTS = {
    "sum_not_mean": ("const double ms = ss / n;", "const double ms = ss;"),
    "eps_outside_sqrt": ("1.0 / sqrt(ms + eps)", "1.0 / (sqrt(ms) + eps)"),
    "no_sqrt": ("1.0 / sqrt(ms + eps)", "1.0 / (ms + eps)"),
    "gain_dropped": ("* inv * widen_bf16(w[c]);", "* inv;"),
    "gain_shifted": ("* inv * widen_bf16(w[c]);", "* inv * widen_bf16(w[(c + 1) % n]);"),
    "abs_not_square": ("ss += v * v;", "ss += fabs(v);"),
    "last_column_skipped": ("for (int c = 0; c < n; ++c) {\n            const double v",
                            "for (int c = 0; c < n - 1; ++c) {\n            const double v"),
}


# The same for the backward oracle.
BWD_MUTANTS = {
    "delta_dropped": ("const double ds = s[j] * (dp[j] - dl);", "const double ds = s[j] * dp[j];"),
    "ds_sign_flipped": ("const double ds = s[j] * (dp[j] - dl);",
                        "const double ds = s[j] * (dl - dp[j]);"),
    "dq_scale_dropped": ("dq[qi + d] += scale * ds *", "dq[qi + d] += ds *"),
    "dk_from_keys": ("dk[kj + d] += scale * ds * wide(q, qi + d);",
                     "dk[kj + d] += scale * ds * wide(k, kj + d);"),
    "dv_from_ds": ("dv[kj + d] += s[j] * wide(dout, qi + d);",
                   "dv[kj + d] += ds * wide(dout, qi + d);"),
    "dp_from_keys": ("dot += wide(dout, qi + d) * wide(v,", "dot += wide(dout, qi + d) * wide(k,"),
    "mask_ignored": ("const int n = causal ? i + 1 : T;", "const int n = T;"),
    "unnormalised": ("s[j] /= Z;", "s[j] /= 1.0;"),
    "rows_key_mask_shifted": ("for (int i = causal ? j : 0; i < T; ++i) {",
                              "for (int i = causal ? j + 1 : 0; i < T; ++i) {"),
    "rows_dv_without_p": ("ov[d] += p * wide(dout, qi + d);", "ov[d] += wide(dout, qi + d);"),
    "rows_delta_unweighted": ("dl += exp(s[j] - lse) * dot;", "dl += dot;"),
    "rows_dq_scale_dropped": ("o[d] += scale * ds * wide(k, kv0", "o[d] += ds * wide(k, kv0"),
}


# The same for the paged-decode oracle.  Every mutant still reads only the
# blocks the table names for the sequence (a wrong block index could read past
# the cache and crash the test process instead of failing a pin).
PAGED_MUTANTS = {
    "interleaved_head_map": ("const int g = h / G;", "const int g = h % Hkv;"),
    "row_shifted_in_block": ("* block_size + t % block_size) * D;",
                             "* block_size + (t + 1) % block_size) * D;"),
    "mask_hides_newest": ("int vis = causal ? n - Tq + i + 1 : n;",
                          "int vis = causal ? n - Tq + i : n;"),
    "mask_ignored": ("int vis = causal ? n - Tq + i + 1 : n;", "int vis = n;"),
    "mask_from_front": ("int vis = causal ? n - Tq + i + 1 : n;",
                        "int vis = causal ? i + 1 : n;"),
    "scale_dropped": ("s[t] = scale * dot;", "s[t] = dot;"),
    "values_from_keys": ("o[d] += w * widen16(v_cache, row + d);",
                         "o[d] += w * widen16(k_cache, row + d);"),
    "lse_without_max": ("= m + log(Z);", "= log(Z);"),
    "empty_row_lse_zero": ("lse[((int64_t)b * Hq + h) * Tq + i] = -INFINITY;",
                           "lse[((int64_t)b * Hq + h) * Tq + i] = 0.0;"),
    "unnormalised": ("const double w = s[t] / Z;", "const double w = s[t];"),
    "query_from_head_zero": ("const int64_t qi = (((int64_t)b * Hq + h) * Tq + i) * D;",
                             "const int64_t qi = (((int64_t)b * Hq + 0 * h) * Tq + i) * D;"),
}


def build_mutant(tmp_path: Path, attn_src: str = None, rms_src: str = None, bwd_src: str = None,
                 paged_src: str = None) -> OracleLib:
    """The oracle library built from the given sources (the real file for each
    one not given)."""
    texts = [(attn_src, SOURCE), (rms_src, RMS_SOURCE), (bwd_src, BWD_SOURCE),
             (paged_src, PAGED_SOURCE)]
    files = []
    for i, (text, real) in enumerate(texts):
        f = tmp_path / f"mutant_{i}.c"
        f.write_text(text if text is not None else real.read_text())
        files.append(str(f))
    so = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99", *files, "-o",
                    str(so), "-lm"], check=True)
    return OracleLib(so)


@pytest.mark.parametrize("name", sorted(PAGED_MUTANTS))
def test_planted_paged_mistake_is_caught(tmp_path: Path, name):
    old, new = PAGED_MUTANTS[name]
    src = PAGED_SOURCE.read_text()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutant = build_mutant(tmp_path, paged_src=src.replace(old, new, 1))
    assert caught_by(mutant, ALL_PAGED_PINS), f"no pin rejects the planted mistake {name}"


@pytest.mark.parametrize("name", sorted(BWD_MUTANTS))
def test_planted_backward_mistake_is_caught(tmp_path: Path, name):
    old, new = BWD_MUTANTS[name]
    src = BWD_SOURCE.read_text()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutant = build_mutant(tmp_path, bwd_src=src.replace(old, new, 1))
    assert caught_by(mutant, ALL_BWD_PINS), f"no pin rejects the planted mistake {name}"


def caught_by(mutant, pins):
    caught = []
    for pin in pins:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, ValueError):
            caught.append(pin.__name__)
    return caught


@pytest.mark.parametrize("name", sorted(RMS_MUTANTS))
def test_planted_rmsnorm_mistake_is_caught(tmp_path: Path, name):
    old, new = RMS_MUTANTS[name]
    src = RMS_SOURCE.read_text()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutant = build_mutant(tmp_path, rms_src=src.replace(old, new, 1))
    assert caught_by(mutant, ALL_RMS_PINS), f"no pin rejects the planted mistake {name}"


@pytest.mark.parametrize("name", sorted(MUTANTS))
def test_planted_mistake_is_caught(tmp_path: Path, name):
    old, new = MUTANTS[name]
    src = SOURCE.read_text()
    assert src.count(old) >= 1, f"mutation anchor for {name} not found"
    mutant = build_mutant(tmp_path, attn_src=src.replace(old, new, 1))
    caught = []
    for pin in ALL_PINS:
        try:
            pin(mutant)
        except (AssertionError, RuntimeError, ValueError):
            caught.append(pin.__name__)
    assert caught, f"no pin rejects the planted mistake {name}"


def test_thread_count_does_not_change_bits(lib):
    q, k, v = rand_inputs(2, 4, 2, 40, 16, "bf16", seed=21)
    O1, l1 = lib.attn_fwd(q, k, v, True, 0.25, nthreads=1)
    O8, l8 = lib.attn_fwd(q, k, v, True, 0.25, nthreads=0)
    assert np.array_equal(O1, O8) and np.array_equal(l1, l8)


def test_argument_errors(lib):
    q, k, v = rand_inputs(1, 4, 2, 8, 4, "fp32", seed=0)
    c = lib.lib
    O = np.empty((1, 4, 8, 4))
    lse = np.empty((1, 4, 8))
    dp = ctypes.POINTER(ctypes.c_double)
    ptr = lambda a: a.ctypes.data_as(ctypes.c_void_p)  # noqa: E731
    args = lambda **kw: [kw.get("q", ptr(q)), ptr(k), ptr(v), kw.get("dtype", 0),  # noqa: E731
                         kw.get("B", 1), kw.get("Hq", 4), kw.get("Hkv", 2), kw.get("T", 8),
                         kw.get("D", 4), kw.get("causal", 1), 0.5,
                         O.ctypes.data_as(dp), lse.ctypes.data_as(dp), 1]
    assert c.tessera_oracle_attn_fwd(*args()) == 0
    assert c.tessera_oracle_attn_fwd(*args(q=None)) == 1
    assert c.tessera_oracle_attn_fwd(*args(dtype=5)) == 2
    assert c.tessera_oracle_attn_fwd(*args(T=0)) == 3
    assert c.tessera_oracle_attn_fwd(*args(Hq=3)) == 4
    assert c.tessera_oracle_attn_fwd(*args(causal=2)) == 5
    with pytest.raises(ValueError):
        lib.attn_fwd(q.astype(np.float64), k, v, True, 0.5)
    with pytest.raises(RuntimeError):
        lib.attn_rows(q, k, v, True, 0.5, np.array([4 * 8], np.int64))


def test_pins_module_is_standalone():
    # the pins must not lean on the HIP package
    text = Path(oracle_pins.__file__).read_text()
    assert "attention_flashattention_fwd_amd" not in text


def test_paged_argument_errors(lib):
    from tests.paged_pins import rand_paged
    q, kc, vc, table, lens = rand_paged(2, 4, 2, 1, 8, 16, [5, 20], seed=3)
    lib.paged_decode(q, kc, vc, table, lens, True, 0.5)
    too_long = lens.copy()
    too_long[1] = table.shape[1] * 16 + 1
    with pytest.raises(RuntimeError):
        lib.paged_decode(q, kc, vc, table, too_long, True, 0.5)
    bad = table.copy()
    bad[1, 1] = kc.shape[0]
    with pytest.raises(RuntimeError):
        lib.paged_decode(q, kc, vc, bad, lens, True, 0.5)
    with pytest.raises(ValueError):
        lib.paged_decode(q, kc, vc[:, :1], table, lens, True, 0.5)
