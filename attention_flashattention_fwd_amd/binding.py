"""Thin ctypes binding over the C ABI in include/*.h (tessera_attn.h,
tessera_attn_bwd.h, tessera_paged.h, tessera_rmsnorm.h).

Argument marshalling only: every step of the attention forward pass runs in
the HIP kernels of libtessera_attn.so.  torch supplies device memory and the
current stream.  There is no fallback: without the built library, or without
a GPU, these functions raise.
"""
from __future__ import annotations

import contextlib
import ctypes
import math
from pathlib import Path

import numpy as np

PKG = Path(__file__).resolve().parent
LIBRARY = PKG / "libtessera_attn.so"
# The LDS-poisoned debug build of the same sources (tests only; see build.py).
POISON_LIBRARY = PKG / "libtessera_attn_poison.so"

# status codes (enum tessera_attn_status)
OK = 0
ERR_NULL = 1
ERR_SHAPE = 2
ERR_UNSUPPORTED = 3
ERR_CAUSAL = 4
ERR_SCALE = 5
ERR_ALIGN = 6
ERR_ALIAS = 7
ERR_TOO_LARGE = 8
ERR_LAUNCH = 9
ERR_EPS = 10
ERR_WORKSPACE = 11
ERR_SCRATCH = 12

EXPORTS = ("tessera_attn_fwd", "tessera_attn_fwd_kv", "tessera_attn_fwd_f32", "tessera_attn_bwd",
           "tessera_attn_status_string", "tessera_attn_last_error", "tessera_attn_version",
           "tessera_rmsnorm_fwd", "tessera_paged_decode", "tessera_paged_decode_workspace",
           "tessera_paged_decode_noalloc", "tessera_paged_decode_scratch_limit",
           "tessera_attn_fwd_tile_config", "tessera_attn_fwd_with_config")


class TileConfig(ctypes.Structure):
    """tessera_attn_tile_config (include/tessera_attn.h)."""
    _fields_ = [("heads_per_workgroup", ctypes.c_int), ("query_rows_per_wave", ctypes.c_int),
                ("workgroups_per_cu", ctypes.c_int), ("persistent", ctypes.c_int)]

    def as_tuple(self):
        return (self.heads_per_workgroup, self.query_rows_per_wave, self.workgroups_per_cu,
                self.persistent)

    def __repr__(self):
        return ("TileConfig(heads_per_workgroup={}, query_rows_per_wave={}, "
                "workgroups_per_cu={}, persistent={})".format(*self.as_tuple()))

_libs: dict[Path, ctypes.CDLL] = {}
_active = LIBRARY


def library_path() -> Path:
    return _active


def _load(path: Path) -> ctypes.CDLL:
    if not path.exists():
        raise RuntimeError(
            f"{path} is missing: build it with "
            "`python -m attention_flashattention_fwd_amd.build` (needs ROCm hipcc)")
    L = ctypes.CDLL(str(path))
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    sig = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.tessera_attn_fwd.argtypes = sig
    L.tessera_attn_fwd.restype = i
    L.tessera_attn_fwd_f32.argtypes = sig
    L.tessera_attn_fwd_f32.restype = i
    L.tessera_attn_fwd_kv.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f, vp]
    L.tessera_attn_fwd_kv.restype = i
    L.tessera_attn_bwd.argtypes = [vp] * 10 + [i] * 6 + [f, vp]
    L.tessera_attn_bwd.restype = i
    L.tessera_rmsnorm_fwd.argtypes = [vp, vp, vp, ctypes.c_longlong, i, f, vp]
    L.tessera_rmsnorm_fwd.restype = i
    L.tessera_paged_decode.argtypes = [vp] * 7 + [i] * 9 + [f, vp, ctypes.c_longlong, vp]
    L.tessera_paged_decode.restype = i
    L.tessera_paged_decode_workspace.argtypes = [i] * 7
    L.tessera_paged_decode_noalloc.argtypes = [vp] * 7 + [i] * 9 + [f, vp]
    L.tessera_paged_decode_noalloc.restype = i
    L.tessera_attn_fwd_tile_config.argtypes = [i] * 7 + [ctypes.POINTER(TileConfig)]
    L.tessera_attn_fwd_tile_config.restype = i
    L.tessera_attn_fwd_with_config.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, f,
                                               ctypes.POINTER(TileConfig), vp]
    L.tessera_attn_fwd_with_config.restype = i
    L.tessera_paged_decode_scratch_limit.argtypes = []
    L.tessera_paged_decode_scratch_limit.restype = ctypes.c_longlong
    L.tessera_paged_decode_workspace.restype = ctypes.c_longlong
    L.tessera_attn_status_string.argtypes = [i]
    L.tessera_attn_status_string.restype = ctypes.c_char_p
    L.tessera_attn_last_error.argtypes = []
    L.tessera_attn_last_error.restype = ctypes.c_char_p
    L.tessera_attn_version.argtypes = []
    L.tessera_attn_version.restype = i
    return L


def lib() -> ctypes.CDLL:
    """The loaded HIP library (the production one unless use_library() says
    otherwise); raises if it has not been built."""
    if _active not in _libs:
        _libs[_active] = _load(_active)
    return _libs[_active]


@contextlib.contextmanager
def use_library(path: Path):
    """Routes every call of this module through the HIP library at `path`
    inside the block (the tests run the LDS-poisoned debug build this way).
    Not thread-safe: the choice is module-wide."""
    global _active
    prev, _active = _active, Path(path)
    try:
        yield lib()
    finally:
        _active = prev


def version() -> int:
    return int(lib().tessera_attn_version())


def status_string(code: int) -> str:
    return lib().tessera_attn_status_string(int(code)).decode()


def raw_fwd(dtype: str, q, k, v, out, lse, B, Hq, Hkv, T, D, causal, scale, stream) -> int:
    """Call the C entry point with integer device addresses; returns the status."""
    fn = lib().tessera_attn_fwd if dtype == "bf16" else lib().tessera_attn_fwd_f32
    return int(fn(q, k, v, out, lse, int(B), int(Hq), int(Hkv), int(T), int(D), int(causal),
                  float(np.float32(scale)), stream))


def raw_fwd_kv(q, k, v, out, lse, B, Hq, Hkv, Tq, Tk, D, causal, scale, stream) -> int:
    """Call tessera_attn_fwd_kv (bf16) with integer device addresses; returns the status."""
    return int(lib().tessera_attn_fwd_kv(q, k, v, out, lse, int(B), int(Hq), int(Hkv), int(Tq),
                                         int(Tk), int(D), int(causal),
                                         float(np.float32(scale)), stream))


def tile_config(B, Hq, Hkv, Tq, Tk, D, causal) -> TileConfig:
    """The tile configuration the library's table picks for these sizes."""
    c = TileConfig()
    st = int(lib().tessera_attn_fwd_tile_config(int(B), int(Hq), int(Hkv), int(Tq), int(Tk),
                                                int(D), int(causal), ctypes.byref(c)))
    if st != OK:
        raise RuntimeError(f"tessera_attn_fwd_tile_config failed ({st}): {status_string(st)}")
    return c


def raw_fwd_with_config(q, k, v, out, lse, B, Hq, Hkv, Tq, Tk, D, causal, scale, config,
                        stream) -> int:
    """Call tessera_attn_fwd_with_config with integer device addresses and a
    TileConfig (or None); returns the status."""
    ptr = ctypes.byref(config) if config is not None else None
    return int(lib().tessera_attn_fwd_with_config(q, k, v, out, lse, int(B), int(Hq), int(Hkv),
                                                  int(Tq), int(Tk), int(D), int(causal),
                                                  float(np.float32(scale)), ptr, stream))


def attn_fwd_with_config_into(q, k, v, out, lse, config: TileConfig, causal: bool = True,
                              scale: float | None = None, stream=None) -> None:
    """attn_fwd_kv_into with an explicit tile configuration (bfloat16 only)."""
    import torch

    B, Hq, Hkv, Tq, D = _check_inputs(q, k, v, same_rows=False)
    Tk = k.shape[2]
    if q.dtype != torch.bfloat16:
        raise ValueError("attn_fwd_with_config takes bfloat16 q, k, v")
    if out.shape != q.shape or out.dtype != q.dtype or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32 or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, Tq]")
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = raw_fwd_with_config(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                 lse.data_ptr(), B, Hq, Hkv, Tq, Tk, D, int(bool(causal)), scale,
                                 config, handle)
    if st != OK:
        msg = status_string(st)
        if st == ERR_LAUNCH:
            msg += ": " + lib().tessera_attn_last_error().decode()
        raise RuntimeError(f"tessera_attn_fwd_with_config failed ({st}): {msg}")


def _check_inputs(q, k, v, same_rows: bool = True):
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise ValueError(f"{name} must be a torch.Tensor")
        if t.device.type != "cuda":
            raise ValueError(f"{name} must be on a GPU device, got {t.device}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, T, D], got shape {tuple(t.shape)}")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if not (q.dtype == k.dtype == v.dtype) or q.dtype not in (torch.bfloat16, torch.float32):
        raise ValueError("q, k, v must all be bfloat16 or all float32")
    if not (q.device == k.device == v.device):
        raise ValueError("q, k, v must be on one device")
    B, Hq, T, D = q.shape
    if k.shape != v.shape or k.shape[0] != B or k.shape[3] != D \
            or (same_rows and k.shape[2] != T):
        rows = "T" if same_rows else "Tk"
        raise ValueError(f"k, v must be [B, Hkv, {rows}, D] with B={B}, D={D}"
                         + (f", T={T}" if same_rows else "")
                         + f"; got {tuple(k.shape)} and {tuple(v.shape)}")
    return B, Hq, k.shape[1], T, D


def attn_fwd_into(q, k, v, out, lse, causal: bool = True, scale: float | None = None,
                  stream=None) -> None:
    """Write attention of (q, k, v) into preallocated `out` [B,Hq,T,D] (q's
    dtype) and `lse` [B,Hq,T] float32.  Enqueued on `stream` (default: the
    current torch stream of q's device); nothing is allocated."""
    import torch

    B, Hq, Hkv, T, D = _check_inputs(q, k, v)
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse.shape != (B, Hq, T) or lse.dtype != torch.float32 or lse.device != q.device \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, T] on q's device")
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    dtype = "bf16" if q.dtype == torch.bfloat16 else "fp32"
    with torch.cuda.device(q.device):
        st = raw_fwd(dtype, q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                     lse.data_ptr(), B, Hq, Hkv, T, D, int(bool(causal)), scale, handle)
    if st != OK:
        msg = status_string(st)
        if st == ERR_LAUNCH:
            msg += ": " + lib().tessera_attn_last_error().decode()
        raise RuntimeError(f"tessera_attn_fwd failed ({st}): {msg}")


def attn_fwd(q, k, v, causal: bool = True, scale: float | None = None):
    """Attention forward.  Returns (out [B,Hq,T,D] in q's dtype, lse [B,Hq,T] float32).

    q [B,Hq,T,D], k/v [B,Hkv,T,D], contiguous, all bfloat16 or all float32,
    on one GPU.  scale defaults to float32(1/sqrt(D))."""
    import torch

    B, Hq, Hkv, T, D = _check_inputs(q, k, v)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    attn_fwd_into(q, k, v, out, lse, causal, scale)
    return out, lse


def attn_fwd_kv_into(q, k, v, out, lse, causal: bool = True, scale: float | None = None,
                     stream=None) -> None:
    """tessera_attn_fwd_kv: q [B,Hq,Tq,D] against the keys and values k, v
    [B,Hkv,Tk,D] (bfloat16), query row i standing at position i + Tk - Tq;
    writes `out` [B,Hq,Tq,D] bfloat16 and `lse` [B,Hq,Tq] float32.  Enqueued on
    `stream` (default: the current torch stream of q's device)."""
    import torch

    B, Hq, Hkv, Tq, D = _check_inputs(q, k, v, same_rows=False)
    Tk = k.shape[2]
    if q.dtype != torch.bfloat16:
        raise ValueError("attn_fwd_kv takes bfloat16 q, k, v")
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32 or lse.device != q.device \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, Tq] on q's device")
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = raw_fwd_kv(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                        lse.data_ptr(), B, Hq, Hkv, Tq, Tk, D, int(bool(causal)), scale, handle)
    if st != OK:
        msg = status_string(st)
        if st == ERR_LAUNCH:
            msg += ": " + lib().tessera_attn_last_error().decode()
        raise RuntimeError(f"tessera_attn_fwd_kv failed ({st}): {msg}")


def attn_fwd_kv(q, k, v, causal: bool = True, scale: float | None = None):
    """Attention of Tq new query rows against Tk cached key/value rows
    (bfloat16).  Returns (out [B,Hq,Tq,D], lse [B,Hq,Tq] float32)."""
    import torch

    B, Hq, Hkv, Tq, D = _check_inputs(q, k, v, same_rows=False)
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    attn_fwd_kv_into(q, k, v, out, lse, causal, scale)
    return out, lse


RMSNORM_EPS = 1e-6   # the default gain-normalisation epsilon (the pages give none)


def raw_rmsnorm(x, w, y, rows, n, eps, stream) -> int:
    """Call tessera_rmsnorm_fwd with integer device addresses; returns the status."""
    return int(lib().tessera_rmsnorm_fwd(x, w, y, int(rows), int(n), float(np.float32(eps)),
                                         stream))


def rmsnorm_fwd_into(x, w, y, eps: float = RMSNORM_EPS, stream=None) -> None:
    """Fused RMSNorm: y = x / sqrt(mean(x^2, last dim) + eps) * w, bfloat16.
    x and y are contiguous [..., n] (y may be x), w is [n]."""
    import torch

    for name, t in (("x", x), ("w", w), ("y", y)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a torch.Tensor on a GPU device")
        if t.dtype != torch.bfloat16 or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous bfloat16 tensor")
    n = x.shape[-1] if x.dim() else 0
    if w.shape != (n,) or y.shape != x.shape or not (x.device == w.device == y.device):
        raise ValueError(f"w must be [{n}] and y shaped like x, all on one device")
    rows = x.numel() // n if n else 0
    if stream is None:
        stream = torch.cuda.current_stream(x.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(x.device):
        st = raw_rmsnorm(x.data_ptr(), w.data_ptr(), y.data_ptr(), rows, n, eps, handle)
    if st != OK:
        msg = status_string(st)
        if st == ERR_LAUNCH:
            msg += ": " + lib().tessera_attn_last_error().decode()
        raise RuntimeError(f"tessera_rmsnorm_fwd failed ({st}): {msg}")


def rmsnorm_fwd(x, w, eps: float = RMSNORM_EPS):
    """Fused RMSNorm of the last dimension of x (bfloat16); returns y like x."""
    import torch

    y = torch.empty_like(x)
    rmsnorm_fwd_into(x, w, y, eps)
    return y


def raw_bwd(q, k, v, out, dout, lse, dq, dk, dv, delta, B, Hq, Hkv, T, D, causal, scale,
            stream) -> int:
    """Call tessera_attn_bwd with integer device addresses; returns the status."""
    return int(lib().tessera_attn_bwd(q, k, v, out, dout, lse, dq, dk, dv, delta, int(B),
                                      int(Hq), int(Hkv), int(T), int(D), int(causal),
                                      float(np.float32(scale)), stream))


def attn_bwd(q, k, v, out, lse, dout, causal: bool = True, scale: float | None = None,
             stream=None):
    """Gradients of attn_fwd (bfloat16): given its inputs, its results out and
    lse, and the output gradient dout, returns (dq, dk, dv, delta), delta
    being the row sums of dout * out [B,Hq,T] float32."""
    import torch

    B, Hq, Hkv, T, D = _check_inputs(q, k, v)
    if q.dtype != torch.bfloat16:
        raise ValueError("attn_bwd takes bfloat16 q, k, v")
    for name, t in (("out", out), ("dout", dout)):
        if t.shape != q.shape or t.dtype != q.dtype or t.device != q.device \
                or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous tensor shaped and typed like q")
    if lse.shape != (B, Hq, T) or lse.dtype != torch.float32 or lse.device != q.device \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, T] on q's device")
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty((B, Hq, T), dtype=torch.float32, device=q.device)
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = raw_bwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), dout.data_ptr(),
                     lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(),
                     delta.data_ptr(), B, Hq, Hkv, T, D, int(bool(causal)), scale, handle)
    if st != OK:
        msg = status_string(st)
        if st == ERR_LAUNCH:
            msg += ": " + lib().tessera_attn_last_error().decode()
        raise RuntimeError(f"tessera_attn_bwd failed ({st}): {msg}")
    return dq, dk, dv, delta


def raw_paged_workspace(B, Hq, Hkv, Tq, D, block_size, max_blocks) -> int:
    """tessera_paged_decode_workspace: bytes needed, or -status."""
    return int(lib().tessera_paged_decode_workspace(int(B), int(Hq), int(Hkv), int(Tq), int(D),
                                                    int(block_size), int(max_blocks)))


def raw_paged(q, kc, vc, table, lens, out, lse, B, Hq, Hkv, Tq, D, num_blocks, block_size,
              max_blocks, causal, scale, ws, ws_bytes, stream) -> int:
    """Call tessera_paged_decode with integer device addresses; returns the status."""
    return int(lib().tessera_paged_decode(q, kc, vc, table, lens, out, lse, int(B), int(Hq),
                                          int(Hkv), int(Tq), int(D), int(num_blocks),
                                          int(block_size), int(max_blocks), int(causal),
                                          float(np.float32(scale)), ws, int(ws_bytes), stream))


def raw_paged_noalloc(q, kc, vc, table, lens, out, lse, B, Hq, Hkv, Tq, D, num_blocks,
                      block_size, max_blocks, causal, scale, stream) -> int:
    """Call tessera_paged_decode_noalloc with integer device addresses; returns
    the status."""
    return int(lib().tessera_paged_decode_noalloc(q, kc, vc, table, lens, out, lse, int(B),
                                                  int(Hq), int(Hkv), int(Tq), int(D),
                                                  int(num_blocks), int(block_size),
                                                  int(max_blocks), int(causal),
                                                  float(np.float32(scale)), stream))


def paged_scratch_limit() -> int:
    """Bytes of the library's fixed scratch behind tessera_paged_decode_noalloc."""
    return int(lib().tessera_paged_decode_scratch_limit())


def _check_paged(q, k_cache, v_cache, block_table, context_lens):
    import torch

    for name, t, dt, nd in (("q", q, torch.bfloat16, 4), ("k_cache", k_cache, torch.bfloat16, 4),
                            ("v_cache", v_cache, torch.bfloat16, 4),
                            ("block_table", block_table, torch.int32, 2),
                            ("context_lens", context_lens, torch.int32, 1)):
        if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
            raise ValueError(f"{name} must be a torch.Tensor on a GPU device")
        if t.dtype != dt or t.dim() != nd or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous {nd}-D {dt} tensor")
        if t.device != q.device:
            raise ValueError("all paged-decode tensors must be on one device")
    B, Hq, Tq, D = q.shape
    num_blocks, Hkv, block_size, Dk = k_cache.shape
    if v_cache.shape != k_cache.shape or Dk != D or block_table.shape[0] != B \
            or context_lens.shape != (B,):
        raise ValueError("q [B,Hq,Tq,D], caches [num_blocks,Hkv,block_size,D], "
                         "block_table [B,max_blocks], context_lens [B]")
    return B, Hq, Hkv, Tq, D, num_blocks, block_size, block_table.shape[1]


def paged_workspace_bytes(B, Hq, Hkv, Tq, D, block_size, max_blocks) -> int:
    """Bytes of workspace tessera_paged_decode needs (raises on bad sizes)."""
    n = raw_paged_workspace(B, Hq, Hkv, Tq, D, block_size, max_blocks)
    if n < 0:
        raise RuntimeError(f"tessera_paged_decode_workspace failed ({-n}): {status_string(-n)}")
    return n


def paged_decode_into(q, k_cache, v_cache, block_table, context_lens, out, lse, workspace,
                      causal: bool = True, scale: float | None = None, stream=None) -> None:
    """Decode attention over a block-paged cache into preallocated out
    [B,Hq,Tq,D] bfloat16 and lse [B,Hq,Tq] float32; `workspace` is a uint8
    tensor of at least paged_workspace_bytes(...) bytes."""
    import torch

    B, Hq, Hkv, Tq, D, nblk, bs, maxb = _check_paged(q, k_cache, v_cache, block_table,
                                                      context_lens)
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32 or lse.device != q.device \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, Tq] on q's device")
    ws, ws_bytes = 0, 0
    if workspace is not None:
        if workspace.device != q.device or not workspace.is_contiguous():
            raise ValueError("workspace must be a contiguous tensor on q's device")
        ws, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = raw_paged(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                       block_table.data_ptr(), context_lens.data_ptr(), out.data_ptr(),
                       lse.data_ptr(), B, Hq, Hkv, Tq, D, nblk, bs, maxb, int(bool(causal)),
                       scale, ws, ws_bytes, handle)
    if st != OK:
        msg = status_string(st)
        if st == ERR_LAUNCH:
            msg += ": " + lib().tessera_attn_last_error().decode()
        raise RuntimeError(f"tessera_paged_decode failed ({st}): {msg}")


def paged_decode_noalloc_into(q, k_cache, v_cache, block_table, context_lens, out, lse,
                              causal: bool = True, scale: float | None = None,
                              stream=None) -> None:
    """paged_decode_into without a workspace: tessera_paged_decode_noalloc,
    whose split partials use the library's fixed per-GPU scratch buffer, so
    neither this call nor the library allocates.  Calls on one GPU must not
    overlap in time (they share that buffer)."""
    import torch

    B, Hq, Hkv, Tq, D, nblk, bs, maxb = _check_paged(q, k_cache, v_cache, block_table,
                                                      context_lens)
    if out.shape != q.shape or out.dtype != q.dtype or out.device != q.device \
            or not out.is_contiguous():
        raise ValueError("out must be a contiguous tensor shaped and typed like q")
    if lse.shape != (B, Hq, Tq) or lse.dtype != torch.float32 or lse.device != q.device \
            or not lse.is_contiguous():
        raise ValueError("lse must be a contiguous float32 tensor [B, Hq, Tq] on q's device")
    if scale is None:
        scale = float(np.float32(1.0 / math.sqrt(D)))
    if stream is None:
        stream = torch.cuda.current_stream(q.device)
    handle = stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)
    with torch.cuda.device(q.device):
        st = raw_paged_noalloc(q.data_ptr(), k_cache.data_ptr(), v_cache.data_ptr(),
                               block_table.data_ptr(), context_lens.data_ptr(), out.data_ptr(),
                               lse.data_ptr(), B, Hq, Hkv, Tq, D, nblk, bs, maxb,
                               int(bool(causal)), scale, handle)
    if st != OK:
        msg = status_string(st)
        if st == ERR_LAUNCH:
            msg += ": " + lib().tessera_attn_last_error().decode()
        raise RuntimeError(f"tessera_paged_decode_noalloc failed ({st}): {msg}")


def paged_decode(q, k_cache, v_cache, block_table, context_lens, causal: bool = True,
                 scale: float | None = None):
    """Attention of the Tq newest tokens of each sequence over its K/V in a
    block-paged cache (layout in include/tessera_paged.h).  Returns
    (out [B,Hq,Tq,D] bfloat16, lse [B,Hq,Tq] float32)."""
    import torch

    B, Hq, Hkv, Tq, D, _, bs, maxb = _check_paged(q, k_cache, v_cache, block_table,
                                                   context_lens)
    n = paged_workspace_bytes(B, Hq, Hkv, Tq, D, bs, maxb)
    ws = torch.empty(n, dtype=torch.uint8, device=q.device) if n else None
    out = torch.empty_like(q)
    lse = torch.empty((B, Hq, Tq), dtype=torch.float32, device=q.device)
    paged_decode_into(q, k_cache, v_cache, block_table, context_lens, out, lse, ws, causal, scale)
    return out, lse
