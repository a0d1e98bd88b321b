"""ctypes wrapper around the plain-C fp64 oracle (attn_oracle.c, rmsnorm_oracle.c,
attn_bwd_oracle.c, paged_oracle.c).

TEST INFRASTRUCTURE ONLY: the tests, the package smoke check and the bench's
CPU-baseline leg use it; the HIP path never does.

Inputs are numpy arrays holding exactly the values the GPU receives:
float32 arrays for fp32 runs, or uint16 arrays carrying bf16 bit patterns.
Outputs are float64.  See attn_oracle.c for the definition computed.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from pathlib import Path

import numpy as np

HERE = Path(__file__).resolve().parent
SOURCE = HERE / "attn_oracle.c"
RMS_SOURCE = HERE / "rmsnorm_oracle.c"
BWD_SOURCE = HERE / "attn_bwd_oracle.c"
PAGED_SOURCE = HERE / "paged_oracle.c"
SOURCES = (SOURCE, RMS_SOURCE, BWD_SOURCE, PAGED_SOURCE)
LIBRARY = HERE / "liboracle_attn.so"

DTYPE_F32 = 0
DTYPE_BF16 = 1

_c_double_p = ctypes.POINTER(ctypes.c_double)
_c_int64_p = ctypes.POINTER(ctypes.c_int64)


def build(sources=SOURCES, output: Path = LIBRARY) -> Path:
    """Compile the oracle sources with gcc (plain -O2, OpenMP) into one shared
    library."""
    cmd = ["gcc", "-O2", "-fopenmp", "-fPIC", "-shared", "-std=c99",
           *[str(x) for x in sources], "-o", str(output) + ".tmp", "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(str(output) + ".tmp", output)
    return output


class OracleLib:
    """One loaded copy of the oracle library (the tests also load mutants)."""

    def __init__(self, path: Path):
        self.path = Path(path)
        lib = ctypes.CDLL(str(self.path))
        common = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                  ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int, ctypes.c_int,
                  ctypes.c_int, ctypes.c_double]
        lib.tessera_oracle_attn_fwd.argtypes = common + [_c_double_p, _c_double_p, ctypes.c_int]
        lib.tessera_oracle_attn_fwd.restype = ctypes.c_int
        lib.tessera_oracle_attn_fwd_kv.argtypes = common[:7] + [ctypes.c_int] + common[7:] + [
            _c_double_p, _c_double_p, ctypes.c_int]
        lib.tessera_oracle_attn_fwd_kv.restype = ctypes.c_int
        lib.tessera_oracle_attn_rows.argtypes = common + [
            _c_int64_p, ctypes.c_int64, _c_double_p, _c_double_p, ctypes.c_int]
        lib.tessera_oracle_attn_rows.restype = ctypes.c_int
        lib.tessera_oracle_attn_probs.argtypes = common + [_c_double_p, _c_double_p, _c_double_p]
        lib.tessera_oracle_attn_probs.restype = ctypes.c_int
        lib.tessera_oracle_rmsnorm.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int64,
                                               ctypes.c_int, ctypes.c_double, _c_double_p]
        lib.tessera_oracle_rmsnorm.restype = ctypes.c_int
        vp, ci = ctypes.c_void_p, ctypes.c_int
        lib.tessera_oracle_attn_bwd.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci,
                                                ctypes.c_double] + [_c_double_p] * 4
        lib.tessera_oracle_attn_bwd.restype = ctypes.c_int
        lib.tessera_oracle_attn_bwd_rows.argtypes = [vp, vp, vp, vp, ci, ci, ci, ci, ci, ci,
                                                     ctypes.c_double, _c_int64_p, ctypes.c_int64,
                                                     _c_int64_p, ctypes.c_int64] + [_c_double_p] * 4
        lib.tessera_oracle_attn_bwd_rows.restype = ctypes.c_int
        lib.tessera_oracle_paged_decode.argtypes = [vp] * 5 + [ci] * 9 + [
            ctypes.c_double, _c_double_p, _c_double_p]
        lib.tessera_oracle_paged_decode.restype = ctypes.c_int
        lib.tessera_oracle_threads.argtypes = [ctypes.c_int]
        lib.tessera_oracle_threads.restype = ctypes.c_int
        self.lib = lib

    # -- helpers -----------------------------------------------------------
    @staticmethod
    def _prep(q, k, v, same_rows=True):
        arrs = [np.ascontiguousarray(a) for a in (q, k, v)]
        dt = arrs[0].dtype
        if any(a.dtype != dt for a in arrs):
            raise ValueError("q, k and v must share one dtype")
        if dt == np.float32:
            code = DTYPE_F32
        elif dt == np.uint16:
            code = DTYPE_BF16
        else:
            raise ValueError(f"oracle takes float32 or uint16 (bf16 bits), got {dt}")
        if arrs[0].ndim != 4 or arrs[1].ndim != 4 or arrs[2].ndim != 4:
            raise ValueError("q, k, v must be 4-D [B, H, T, D]")
        B, Hq, T, D = arrs[0].shape
        if arrs[1].shape != arrs[2].shape or arrs[1].shape[0] != B or \
                (same_rows and arrs[1].shape[2] != T) or arrs[1].shape[3] != D:
            raise ValueError("k and v must be [B, Hkv, T, D] matching q")
        Hkv = arrs[1].shape[1]
        return arrs, code, (B, Hq, Hkv, T, D)

    @staticmethod
    def _ptr(a):
        return a.ctypes.data_as(ctypes.c_void_p)

    @staticmethod
    def _check(rc, name):
        if rc != 0:
            raise RuntimeError(f"{name} failed with code {rc}")

    # -- entry points ------------------------------------------------------
    def attn_fwd(self, q, k, v, causal: bool, scale: float, nthreads: int = 0):
        (q, k, v), code, (B, Hq, Hkv, T, D) = self._prep(q, k, v)
        O = np.empty((B, Hq, T, D), np.float64)
        lse = np.empty((B, Hq, T), np.float64)
        rc = self.lib.tessera_oracle_attn_fwd(
            self._ptr(q), self._ptr(k), self._ptr(v), code, B, Hq, Hkv, T, D,
            int(bool(causal)), float(scale),
            O.ctypes.data_as(_c_double_p), lse.ctypes.data_as(_c_double_p), int(nthreads))
        self._check(rc, "tessera_oracle_attn_fwd")
        return O, lse

    def attn_fwd_kv(self, q, k, v, causal: bool, scale: float, nthreads: int = 0):
        """q [B,Hq,Tq,D] against k, v [B,Hkv,Tk,D]; query row i stands at position
        i + Tk - Tq.  Returns O [B,Hq,Tq,D], lse [B,Hq,Tq]."""
        (q, k, v), code, (B, Hq, Hkv, Tq, D) = self._prep(q, k, v, same_rows=False)
        Tk = k.shape[2]
        O = np.empty((B, Hq, Tq, D), np.float64)
        lse = np.empty((B, Hq, Tq), np.float64)
        rc = self.lib.tessera_oracle_attn_fwd_kv(
            self._ptr(q), self._ptr(k), self._ptr(v), code, B, Hq, Hkv, Tq, Tk, D,
            int(bool(causal)), float(scale),
            O.ctypes.data_as(_c_double_p), lse.ctypes.data_as(_c_double_p), int(nthreads))
        self._check(rc, "tessera_oracle_attn_fwd_kv")
        return O, lse

    def attn_rows(self, q, k, v, causal: bool, scale: float, rows, nthreads: int = 0):
        """rows: flat indices (b*Hq + h)*T + i.  Returns O [n, D], lse [n]."""
        (q, k, v), code, (B, Hq, Hkv, T, D) = self._prep(q, k, v)
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.shape[0]
        O = np.empty((n, D), np.float64)
        lse = np.empty((n,), np.float64)
        rc = self.lib.tessera_oracle_attn_rows(
            self._ptr(q), self._ptr(k), self._ptr(v), code, B, Hq, Hkv, T, D,
            int(bool(causal)), float(scale), rows.ctypes.data_as(_c_int64_p), n,
            O.ctypes.data_as(_c_double_p), lse.ctypes.data_as(_c_double_p), int(nthreads))
        self._check(rc, "tessera_oracle_attn_rows")
        return O, lse

    def attn_probs(self, q, k, v, causal: bool, scale: float):
        (q, k, v), code, (B, Hq, Hkv, T, D) = self._prep(q, k, v)
        O = np.empty((B, Hq, T, D), np.float64)
        lse = np.empty((B, Hq, T), np.float64)
        P = np.empty((B, Hq, T, T), np.float64)
        rc = self.lib.tessera_oracle_attn_probs(
            self._ptr(q), self._ptr(k), self._ptr(v), code, B, Hq, Hkv, T, D,
            int(bool(causal)), float(scale), O.ctypes.data_as(_c_double_p),
            lse.ctypes.data_as(_c_double_p), P.ctypes.data_as(_c_double_p))
        self._check(rc, "tessera_oracle_attn_probs")
        return O, lse, P

    def rmsnorm(self, x, w, eps: float):
        """x [rows, n] and w [n] as uint16 bf16 patterns; returns y [rows, n] fp64."""
        x = np.ascontiguousarray(x)
        w = np.ascontiguousarray(w)
        if x.dtype != np.uint16 or w.dtype != np.uint16:
            raise ValueError("rmsnorm oracle takes uint16 bf16 patterns")
        if x.ndim != 2 or w.ndim != 1 or w.shape[0] != x.shape[1]:
            raise ValueError("x must be [rows, n] and w [n]")
        y = np.empty(x.shape, np.float64)
        rc = self.lib.tessera_oracle_rmsnorm(self._ptr(x), self._ptr(w), x.shape[0], x.shape[1],
                                             float(eps), y.ctypes.data_as(_c_double_p))
        self._check(rc, "tessera_oracle_rmsnorm")
        return y

    def attn_bwd(self, q, k, v, dout, causal: bool, scale: float):
        """Gradients of the attention forward for output gradient dout (all uint16
        bf16 patterns; q, dout [B,Hq,T,D], k, v [B,Hkv,T,D]).  Returns dq, dk, dv
        and Delta [B,Hq,T], fp64."""
        (q, k, v), code, (B, Hq, Hkv, T, D) = self._prep(q, k, v)
        dout = np.ascontiguousarray(dout)
        if code != DTYPE_BF16 or dout.dtype != np.uint16 or dout.shape != q.shape:
            raise ValueError("attn_bwd takes bf16 patterns, dout shaped like q")
        dq = np.empty(q.shape, np.float64)
        dk = np.empty(k.shape, np.float64)
        dv = np.empty(v.shape, np.float64)
        delta = np.empty((B, Hq, T), np.float64)
        rc = self.lib.tessera_oracle_attn_bwd(
            self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(dout), B, Hq, Hkv, T, D,
            int(bool(causal)), float(scale), *(a.ctypes.data_as(_c_double_p)
                                               for a in (dq, dk, dv, delta)))
        self._check(rc, "tessera_oracle_attn_bwd")
        return dq, dk, dv, delta

    def attn_bwd_rows(self, q, k, v, dout, causal: bool, scale: float, qrows, krows):
        """The backward's dq and Delta of query rows `qrows` (flat index
        (b*Hq + h)*T + i) and dk, dv of key rows `krows` (flat index
        (b*Hkv + g)*T + j), each from the definitions.  Returns
        (dq [nq,D], delta [nq], dk [nk,D], dv [nk,D]), fp64."""
        (q, k, v), code, (B, Hq, Hkv, T, D) = self._prep(q, k, v)
        dout = np.ascontiguousarray(dout)
        if code != DTYPE_BF16 or dout.dtype != np.uint16 or dout.shape != q.shape:
            raise ValueError("attn_bwd_rows takes bf16 patterns, dout shaped like q")
        qrows = np.ascontiguousarray(qrows, dtype=np.int64)
        krows = np.ascontiguousarray(krows, dtype=np.int64)
        nq, nk = qrows.shape[0], krows.shape[0]
        dq = np.empty((nq, D), np.float64)
        delta = np.empty((nq,), np.float64)
        dk = np.empty((nk, D), np.float64)
        dv = np.empty((nk, D), np.float64)
        rc = self.lib.tessera_oracle_attn_bwd_rows(
            self._ptr(q), self._ptr(k), self._ptr(v), self._ptr(dout), B, Hq, Hkv, T, D,
            int(bool(causal)), float(scale), qrows.ctypes.data_as(_c_int64_p), nq,
            krows.ctypes.data_as(_c_int64_p), nk,
            *(a.ctypes.data_as(_c_double_p) for a in (dq, delta, dk, dv)))
        self._check(rc, "tessera_oracle_attn_bwd_rows")
        return dq, delta, dk, dv

    def paged_decode(self, q, k_cache, v_cache, block_table, context_lens, causal: bool,
                     scale: float):
        """Attention of the Tq newest query rows of each sequence over its K/V
        held in a block-paged cache.  q [B,Hq,Tq,D] and the caches
        [num_blocks,Hkv,block_size,D] are uint16 bf16 patterns; block_table
        [B,max_blocks] and context_lens [B] are int32.  Returns O [B,Hq,Tq,D]
        and lse [B,Hq,Tq], fp64 (rows that see no token: O = 0, lse = -inf)."""
        q, kc, vc = (np.ascontiguousarray(a) for a in (q, k_cache, v_cache))
        bt = np.ascontiguousarray(block_table, dtype=np.int32)
        cl = np.ascontiguousarray(context_lens, dtype=np.int32)
        if q.dtype != np.uint16 or kc.dtype != np.uint16 or vc.dtype != np.uint16:
            raise ValueError("paged_decode takes uint16 bf16 patterns")
        if q.ndim != 4 or kc.ndim != 4 or kc.shape != vc.shape or bt.ndim != 2 or cl.ndim != 1:
            raise ValueError("q [B,Hq,Tq,D], caches [num_blocks,Hkv,block_size,D], "
                             "block_table [B,max_blocks], context_lens [B]")
        B, Hq, Tq, D = q.shape
        num_blocks, Hkv, block_size, Dk = kc.shape
        if Dk != D or bt.shape[0] != B or cl.shape[0] != B:
            raise ValueError("inconsistent paged-decode shapes")
        O = np.empty((B, Hq, Tq, D), np.float64)
        lse = np.empty((B, Hq, Tq), np.float64)
        rc = self.lib.tessera_oracle_paged_decode(
            self._ptr(q), self._ptr(kc), self._ptr(vc), self._ptr(bt), self._ptr(cl), B, Hq, Hkv,
            Tq, D, block_size, bt.shape[1], num_blocks, int(bool(causal)), float(scale),
            O.ctypes.data_as(_c_double_p), lse.ctypes.data_as(_c_double_p))
        self._check(rc, "tessera_oracle_paged_decode")
        return O, lse

    def threads(self, nthreads: int = 0) -> int:
        return int(self.lib.tessera_oracle_threads(int(nthreads)))


_DEFAULT: OracleLib | None = None


def load() -> OracleLib:
    """The oracle built from attn_oracle.c (compiled on first use if absent)."""
    global _DEFAULT
    if _DEFAULT is None:
        newest = max(src.stat().st_mtime for src in SOURCES)
        if not LIBRARY.exists() or LIBRARY.stat().st_mtime < newest:
            build()
        _DEFAULT = OracleLib(LIBRARY)
    return _DEFAULT


def attn_fwd(q, k, v, causal, scale, nthreads=0):
    return load().attn_fwd(q, k, v, causal, scale, nthreads)


def attn_fwd_kv(q, k, v, causal, scale, nthreads=0):
    return load().attn_fwd_kv(q, k, v, causal, scale, nthreads)


def attn_rows(q, k, v, causal, scale, rows, nthreads=0):
    return load().attn_rows(q, k, v, causal, scale, rows, nthreads)


def attn_probs(q, k, v, causal, scale):
    return load().attn_probs(q, k, v, causal, scale)


def attn_bwd(q, k, v, dout, causal, scale):
    return load().attn_bwd(q, k, v, dout, causal, scale)


def attn_bwd_rows(q, k, v, dout, causal, scale, qrows, krows):
    return load().attn_bwd_rows(q, k, v, dout, causal, scale, qrows, krows)


def paged_decode(q, k_cache, v_cache, block_table, context_lens, causal, scale):
    return load().paged_decode(q, k_cache, v_cache, block_table, context_lens, causal, scale)


def rmsnorm(x, w, eps):
    return load().rmsnorm(x, w, eps)


def threads(nthreads=0):
    return load().threads(nthreads)
