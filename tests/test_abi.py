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


def test_status_strings():
    for code in range(0, 12):
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


def test_paged_workspace_sizes():
    # the serving batch: 64 x 8 (sequence, KV head) pairs of up to 16384 tokens
    # -> splits of 1024 keys (64 blocks of 16, the most one split may span),
    # 16 per sequence; 2048 query rows
    cells = 64 * 32 * 1 * 16
    assert binding.raw_paged_workspace(64, 32, 8, 1, 128, 16, 1024) == cells * 4 + cells * 128 * 4
    # short sequences fit one split: no workspace
    assert binding.raw_paged_workspace(2, 4, 2, 1, 64, 16, 8) == 0
    # 1600 tokens in splits of 256: 7 per sequence; the lse part rounds up to 256 bytes
    cells = 1 * 8 * 2 * 7
    assert binding.raw_paged_workspace(1, 8, 2, 2, 32, 16, 100) == 512 + cells * 32 * 4
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
