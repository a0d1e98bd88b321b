"""CPU tests of the C-ABI library: it loads, exports what the header declares,
and rejects bad arguments before touching the GPU (no compute call here)."""
import re
from pathlib import Path

import pytest

from attention_flashattention_fwd_amd import binding

ROOT = Path(__file__).resolve().parent.parent
HEADERS = sorted((ROOT / "include").glob("*.h"))

# fake, well separated, 16-byte aligned device addresses: validation rejects
# these calls before any HIP call is made, so they are never dereferenced
Q, K, V, O, L = (1 << 44), (2 << 44), (3 << 44), (4 << 44), (5 << 44)


def declared_functions():
    names = set()
    for h in HEADERS:
        names |= set(re.findall(r"^\s*(?:const\s+)?(?:\w+\s+)*?\w+\s*\*?\s*(tessera_\w+)\s*\(",
                                h.read_text(), re.M))
    return sorted(names)


def test_header_declares_the_exports():
    assert declared_functions() == sorted(binding.EXPORTS)


def test_library_loads_and_exports_every_symbol():
    lib = binding.lib()
    for name in declared_functions():
        assert hasattr(lib, name), name
    assert binding.version() == 10200


def test_poison_build_loads_and_exports_every_symbol():
    # the LDS-poisoned debug build of the same sources
    with binding.use_library(binding.POISON_LIBRARY) as lib:
        for name in declared_functions():
            assert hasattr(lib, name), name
        assert binding.version() == 10200
        assert call(B=0) == binding.ERR_SHAPE
    assert binding.lib()._name == str(binding.LIBRARY)


def test_status_strings():
    for code in range(0, 13):
        assert binding.status_string(code)
    assert binding.status_string(123) == "unknown status"
    assert binding.lib().tessera_attn_last_error() == b""


def call(dtype="bf16", q=Q, k=K, v=V, o=O, l=L, B=1, Hq=4, Hkv=2, T=64, D=64, causal=1,
         scale=0.125):
    return binding.raw_fwd(dtype, q, k, v, o, l, B, Hq, Hkv, T, D, causal, scale, None)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("kwargs,code", [
    (dict(q=None), binding.ERR_NULL),
    (dict(l=None), binding.ERR_NULL),
    (dict(B=0), binding.ERR_SHAPE),
    (dict(T=0), binding.ERR_SHAPE),
    (dict(Hkv=0), binding.ERR_SHAPE),
    (dict(Hq=3), binding.ERR_SHAPE),
    (dict(D=48), binding.ERR_UNSUPPORTED),
    (dict(D=256), binding.ERR_UNSUPPORTED),
    (dict(causal=2), binding.ERR_CAUSAL),
    (dict(scale=float("nan")), binding.ERR_SCALE),
    (dict(scale=float("inf")), binding.ERR_SCALE),
    (dict(q=Q + 8), binding.ERR_ALIGN),
    (dict(o=O + 2), binding.ERR_ALIGN),
    (dict(l=L + 2), binding.ERR_ALIGN),
    (dict(o=Q), binding.ERR_ALIAS),
    (dict(l=V + 64), binding.ERR_ALIAS),
    (dict(l=O), binding.ERR_ALIAS),
    (dict(B=1 << 16, Hq=1 << 15, Hkv=1 << 15, T=1), binding.ERR_TOO_LARGE),
])
def test_bad_arguments_are_rejected_before_launch(dtype, kwargs, code):
    assert call(dtype, **kwargs) == code


def test_binding_rejects_cpu_tensors():
    import torch
    q = torch.zeros(1, 2, 8, 32, dtype=torch.bfloat16)
    k = torch.zeros(1, 1, 8, 32, dtype=torch.bfloat16)
    with pytest.raises(ValueError, match="GPU"):
        binding.attn_fwd(q, k, k)


def call_kv(q=Q, k=K, v=V, o=O, l=L, B=1, Hq=4, Hkv=2, Tq=16, Tk=64, D=64, causal=1,
            scale=0.125):
    return binding.raw_fwd_kv(q, k, v, o, l, B, Hq, Hkv, Tq, Tk, D, causal, scale, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(k=None), binding.ERR_NULL),
    (dict(Tq=0), binding.ERR_SHAPE),
    (dict(Tk=0), binding.ERR_SHAPE),
    (dict(Tq=65), binding.ERR_SHAPE),                 # causal with more query than key rows
    (dict(D=96), binding.ERR_UNSUPPORTED),
    (dict(causal=-1), binding.ERR_CAUSAL),
    (dict(scale=float("nan")), binding.ERR_SCALE),
    (dict(v=V + 4), binding.ERR_ALIGN),
    (dict(o=K + 1024), binding.ERR_ALIAS),
])
def test_kv_bad_arguments_are_rejected_before_launch(kwargs, code):
    assert call_kv(**kwargs) == code


X, W, Y = (6 << 44), (7 << 44), (8 << 44)


def call_rms(x=X, w=W, y=Y, rows=4, n=64, eps=1e-6):
    return binding.raw_rmsnorm(x, w, y, rows, n, eps, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(x=None), binding.ERR_NULL),
    (dict(w=None), binding.ERR_NULL),
    (dict(rows=0), binding.ERR_SHAPE),
    (dict(n=0), binding.ERR_SHAPE),
    (dict(n=12), binding.ERR_UNSUPPORTED),
    (dict(n=65544), binding.ERR_UNSUPPORTED),
    (dict(eps=-1.0), binding.ERR_EPS),
    (dict(eps=float("nan")), binding.ERR_EPS),
    (dict(x=X + 8), binding.ERR_ALIGN),
    (dict(y=X + 16), binding.ERR_ALIAS),              # partial overlap with x
    (dict(y=W), binding.ERR_ALIAS),
    (dict(rows=1 << 60, n=64), binding.ERR_TOO_LARGE),
])
def test_rmsnorm_bad_arguments_are_rejected_before_launch(kwargs, code):
    assert call_rms(**kwargs) == code


DO, DQ, DK, DV, DL = (9 << 44), (10 << 44), (11 << 44), (12 << 44), (13 << 44)


def call_bwd(q=Q, k=K, v=V, o=O, do=DO, l=L, dq=DQ, dk=DK, dv=DV, dl=DL, B=1, Hq=4, Hkv=2,
             T=64, D=64, causal=1, scale=0.125):
    return binding.raw_bwd(q, k, v, o, do, l, dq, dk, dv, dl, B, Hq, Hkv, T, D, causal, scale,
                           None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(do=None), binding.ERR_NULL),
    (dict(dl=None), binding.ERR_NULL),
    (dict(T=0), binding.ERR_SHAPE),
    (dict(Hq=3), binding.ERR_SHAPE),
    (dict(D=80), binding.ERR_UNSUPPORTED),
    (dict(causal=3), binding.ERR_CAUSAL),
    (dict(scale=float("inf")), binding.ERR_SCALE),
    (dict(dk=DK + 8), binding.ERR_ALIGN),
    (dict(dl=DL + 2), binding.ERR_ALIGN),
    (dict(dq=Q), binding.ERR_ALIAS),                # an output over an input
    (dict(dv=DK + 64), binding.ERR_ALIAS),          # two outputs overlapping
    (dict(dl=DO), binding.ERR_ALIAS),
])
def test_bwd_bad_arguments_are_rejected_before_launch(kwargs, code):
    assert call_bwd(**kwargs) == code


def paged_layout_bytes(B, Hq, Hkv, Tq, D, block_size, max_blocks):
    """The workspace layout written out: per KV head, one slot per decode wave
    (1536 waves in all, 2048 at D=32, no more than the tiles a head can have) plus one per
    sequence; an fp32 log2-sum-exp and an fp32 row of D per query row of the
    head in each slot; two ints per (sequence, KV head)."""
    r256 = lambda x: (x + 255) // 256 * 256  # noqa: E731
    waves = 2048 if D == 32 else 1536
    wg = max(1, min(waves // Hkv, B * ((max_blocks * block_size + 31) // 32)))
    cells = Hkv * (wg + B) * (Hq // Hkv) * Tq
    return r256(cells * 4) + cells * D * 4 + r256(B * Hkv * 8)


def test_paged_workspace_sizes():
    # the serving batch: 192 waves per KV head, 256 slots, 4 query rows each
    assert binding.raw_paged_workspace(64, 32, 8, 1, 128, 16, 1024) == 32768 + 4194304 + 4096
    # short sequences: at most 8 tiles per head -> 8 waves, 10 slots
    assert binding.raw_paged_workspace(2, 4, 2, 1, 64, 16, 8) == 256 + 10240 + 256
    # 1600 tokens: 50 tiles -> 50 waves, 51 slots of 8 rows; the lse part rounds up
    assert binding.raw_paged_workspace(1, 8, 2, 2, 32, 16, 100) == 3328 + 104448 + 256
    for shape in [(64, 32, 8, 1, 128, 16, 1024), (2, 4, 2, 1, 64, 16, 8), (1, 8, 2, 2, 32, 16, 100),
                  (3, 8, 1, 4, 64, 32, 7), (1, 64, 64, 1, 128, 16, 4096),
                  (64, 32, 8, 1, 32, 16, 1024), (2, 8, 1, 1, 32, 16, 4096)]:
        assert binding.raw_paged_workspace(*shape) == paged_layout_bytes(*shape), shape
    assert binding.raw_paged_workspace(1, 8, 2, 9, 32, 16, 100) == -binding.ERR_UNSUPPORTED
    assert binding.raw_paged_workspace(1, 8, 2, 1, 32, 24, 100) == -binding.ERR_UNSUPPORTED
    assert binding.raw_paged_workspace(1, 8, 3, 1, 32, 16, 100) == -binding.ERR_SHAPE
    assert binding.raw_paged_workspace(1, 8, 2, 1, 32, 16, 1 << 28) == -binding.ERR_TOO_LARGE


KC, VC, BT, CL, WS = (14 << 44), (15 << 44), (16 << 44), (17 << 44), (18 << 44)


def call_paged(q=Q, kc=KC, vc=VC, bt=BT, cl=CL, o=O, l=L, B=2, Hq=8, Hkv=2, Tq=2, D=64,
               num_blocks=64, block_size=16, max_blocks=100, causal=1, scale=0.125, ws=WS,
               ws_bytes=1 << 20):
    return binding.raw_paged(q, kc, vc, bt, cl, o, l, B, Hq, Hkv, Tq, D, num_blocks, block_size,
                             max_blocks, causal, scale, ws, ws_bytes, None)


@pytest.mark.parametrize("kwargs,code", [
    (dict(bt=None), binding.ERR_NULL),
    (dict(cl=None), binding.ERR_NULL),
    (dict(num_blocks=0), binding.ERR_SHAPE),
    (dict(max_blocks=0), binding.ERR_SHAPE),
    (dict(Hq=6, Hkv=4), binding.ERR_SHAPE),
    (dict(D=96), binding.ERR_UNSUPPORTED),
    (dict(Tq=9), binding.ERR_UNSUPPORTED),           # 4 heads x 9 rows > 32
    (dict(block_size=8), binding.ERR_UNSUPPORTED),
    (dict(causal=2), binding.ERR_CAUSAL),
    (dict(scale=float("nan")), binding.ERR_SCALE),
    (dict(kc=KC + 8), binding.ERR_ALIGN),
    (dict(ws=WS + 4), binding.ERR_ALIGN),
    (dict(cl=CL + 2), binding.ERR_ALIGN),
    (dict(max_blocks=1 << 28), binding.ERR_TOO_LARGE),
    (dict(ws=None), binding.ERR_WORKSPACE),
    (dict(ws_bytes=100), binding.ERR_WORKSPACE),
    (dict(o=KC + 4096), binding.ERR_ALIAS),         # out inside the K cache
    (dict(l=BT), binding.ERR_ALIAS),
    (dict(ws=CL), binding.ERR_ALIAS),
    (dict(ws=O + 1024), binding.ERR_ALIAS),          # workspace over out
])
def test_paged_bad_arguments_are_rejected_before_launch(kwargs, code):
    assert call_paged(**kwargs) == code


def call_paged_noalloc(q=Q, kc=KC, vc=VC, bt=BT, cl=CL, o=O, l=L, B=2, Hq=8, Hkv=2, Tq=2, D=64,
                       num_blocks=64, block_size=16, max_blocks=100, causal=1, scale=0.125):
    return binding.raw_paged_noalloc(q, kc, vc, bt, cl, o, l, B, Hq, Hkv, Tq, D, num_blocks,
                                     block_size, max_blocks, causal, scale, None)


def test_paged_noalloc_scratch_limit():
    assert binding.paged_scratch_limit() == 32 << 20
    # the serving batch of the bench (64 sequences of up to 16384 tokens) fits
    assert 0 < binding.raw_paged_workspace(64, 32, 8, 1, 128, 16, 1024) <= 32 << 20


@pytest.mark.parametrize("kwargs,code", [
    (dict(bt=None), binding.ERR_NULL),
    (dict(o=None), binding.ERR_NULL),
    (dict(num_blocks=0), binding.ERR_SHAPE),
    (dict(Hq=6, Hkv=4), binding.ERR_SHAPE),
    (dict(D=96), binding.ERR_UNSUPPORTED),
    (dict(block_size=8), binding.ERR_UNSUPPORTED),
    (dict(causal=2), binding.ERR_CAUSAL),
    (dict(scale=float("inf")), binding.ERR_SCALE),
    (dict(kc=KC + 8), binding.ERR_ALIGN),
    (dict(o=KC + 4096), binding.ERR_ALIAS),
    # 32 query rows per KV head in 8 x 256 slots: 34 MB of workspace > 32 MiB
    (dict(B=64, Hq=256, Hkv=8, Tq=1, D=128, max_blocks=4096), binding.ERR_SCRATCH),
])
def test_paged_noalloc_bad_arguments_are_rejected_before_launch(kwargs, code):
    # every check, the scratch limit included, comes before any HIP call
    assert call_paged_noalloc(**kwargs) == code
    assert "scratch" in binding.status_string(binding.ERR_SCRATCH)


def test_tile_table_is_the_sweeps_winners():
    """The table compiled into the library (csrc/tile_table.inc) holds exactly
    the winners that the committed sweep (profiles/tile_sweep_attn_fwd_bf16.md)
    recorded, and each winner is the fastest configuration of its section."""
    import re

    from attention_flashattention_fwd_amd import autotune
    table = autotune.parse_table(
        (ROOT / "attention_flashattention_fwd_amd" / "csrc" / "tile_table.inc").read_text())
    report = (ROOT / "profiles" / "tile_sweep_attn_fwd_bf16.md").read_text()
    recorded = sorted(tuple(int(x) for x in m.group(1).split(","))
                      for m in re.finditer(r"^\s+rule: ([\d, ]+)$", report, re.M))
    assert table == recorded and len(table) == 12
    for sec in re.split(r"^## ", report, flags=re.M)[1:]:
        m = re.match(r"D=(\d+), causal=(\d), (large|small)", sec)
        if not m:
            continue
        timings = [(float(t), tuple(int(x) for x in c.split(",")), "winner" in w)
                   for c, w, t in re.findall(r"^\| \(([\d, ]+)\)( \*\*winner\*\*)? \| ([\d.]+) \|",
                                             sec, re.M)]
        best = min(timings)
        assert best[2], sec.splitlines()[0]
        key = (int(m.group(1)), int(m.group(2)), int(m.group(3) == "large"))
        assert key + best[1] in table


def test_table_picks_fit_the_sizes():
    # the pick for a GQA group of 3 falls back to one head per workgroup, and a
    # ragged key count to one workgroup per CU
    c = binding.tile_config(2, 6, 2, 200, 200, 64, 1)
    assert c.heads_per_workgroup == 1
    c = binding.tile_config(16, 16, 4, 4095, 4095, 64, 1)
    assert c.workgroups_per_cu == 1
    with pytest.raises(RuntimeError):
        binding.tile_config(1, 4, 2, 10, 10, 96, 1)


def test_phase_probe_instruments_the_current_kernel_source():
    """Every anchor of the per-phase timing tool is found once in the kernel
    source, so the instrumented build follows the kernel as it changes."""
    from attention_flashattention_fwd_amd import phase_probe
    text = phase_probe.instrumented_source(phase_probe.SOURCE.read_text())
    assert text.count("__builtin_amdgcn_s_memtime") == 4
    assert "tessera_probe_set" in text


def test_phase_probe_analysis_of_synthetic_records():
    """The probe's summary on hand-made records: 4 items on 2 CUs of 2 XCDs,
    item i with 10 (i + 1) tiles, start 0 and duration 5 + 2 x tiles us
    (timestamps at 100 MHz), steady-state phase cycles 300 / 200 per tile."""
    import numpy as np

    from attention_flashattention_fwd_amd import phase_probe
    items = 4
    rec = np.zeros((items, 8, phase_probe.WORDS), dtype=np.uint32)
    for it in range(items):
        tiles = 10 * (it + 1)
        cu, xcd = it % 2, it // 2          # items 0, 2 share CU 0; 1, 3 CU 1
        start = 0 if it < 2 else 100 * (5 + 2 * 10 * (it - 1))   # second item after the first
        end = start + 100 * (5 + 2 * tiles)
        for w in range(8):
            rec[it, w, 0] = (cu << 8)       # HW_ID: CU id, SH 0, SE 0
            rec[it, w, 8] = 0               # every item on XCD 0 here
            rec[it, w, 1], rec[it, w, 2] = start, 0
            rec[it, w, 3], rec[it, w, 4] = end, 0
            steady = tiles - 4
            rec[it, w, 5] = 300 * steady
            rec[it, w, 7] = 200 * steady
            rec[it, w, 9] = steady | (tiles << 16)
    out = phase_probe.analyse(rec, items)
    assert out["items"] == 4 and out["cus"] == 2
    assert abs(out["item_fixed_us"] - 5.0) < 1e-9 and abs(out["item_us_per_tile"] - 2.0) < 1e-9
    assert out["leading_mfma_phase_cycles_per_tile"] == 300.0
    assert out["lagging_vector_phase_cycles_per_tile"] == 200.0
    assert out["items_per_cu_min_max"] == [2, 2]
    assert out["tiles_per_cu_min_median_max"] == [40, 50.0, 60]   # 10 + 30, 20 + 40
    ends = [e for e in out["cu_last_end_us_min_median_max"]]
    # CU 0: item 2 starts at 25 us (after item 0's 5 + 20), ends at 25 + 65 = 90
    # CU 1: item 3 starts at 45 us, ends at 45 + 85 = 130
    assert abs(ends[0] - 90.0) < 1e-9 and abs(ends[2] - 130.0) < 1e-9
    assert abs(out["span_us"] - 130.0) < 1e-9
