"""Pins of the fp64 RMSNorm oracle to facts other than itself.

Each `pin_*` takes a loaded oracle library and raises AssertionError when the
oracle breaks the fact it checks: brute force at 50 digits on tiny rows,
torch's rms_norm in float64 (an independent library routine), invariance of
the result under scaling a row by a power of two (eps = 0), unit root mean
square of the output when the gain is one, and the closed form of a constant
row.
"""
from __future__ import annotations

import mpmath
import numpy as np
import torch


def bf16_bits(a: np.ndarray) -> np.ndarray:
    """float32 values rounded to bf16 (nearest even), as uint16 patterns."""
    return torch.from_numpy(np.ascontiguousarray(a, np.float32)).to(torch.bfloat16) \
        .view(torch.int16).numpy().view(np.uint16)


def bits_values(b: np.ndarray) -> np.ndarray:
    """uint16 bf16 patterns as float64 values (exact)."""
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def rand_rows(rows, n, seed, scale=1.0):
    rng = np.random.default_rng(seed)
    x = bf16_bits(rng.standard_normal((rows, n), dtype=np.float32) * np.float32(scale))
    w = bf16_bits(1.0 + 0.5 * rng.standard_normal(n, dtype=np.float32))
    return x, w


def pin_rms_mpmath(lib):
    mpmath.mp.dps = 50
    for n_, (rows, n, eps) in enumerate([(1, 1, 0.0), (2, 3, 1e-6), (3, 8, 0.25), (1, 17, 1e-3)]):
        x, w = rand_rows(rows, n, seed=600 + n_)
        y = lib.rmsnorm(x, w, eps)
        xv, wv = bits_values(x), bits_values(w)
        for r in range(rows):
            ms = mpmath.fsum(mpmath.mpf(a) ** 2 for a in xv[r]) / n
            inv = 1 / mpmath.sqrt(ms + mpmath.mpf(eps))
            for c in range(n):
                want = float(mpmath.mpf(xv[r, c]) * inv * mpmath.mpf(wv[c]))
                assert abs(y[r, c] - want) <= 1e-13 * max(1.0, abs(want)), (rows, n, r, c)


def pin_rms_torch(lib):
    for n_, (rows, n, eps) in enumerate([(5, 64, 1e-6), (3, 4096, 1e-5), (2, 24, 0.0)]):
        x, w = rand_rows(rows, n, seed=700 + n_, scale=3.0)
        y = lib.rmsnorm(x, w, eps)
        ref = torch.nn.functional.rms_norm(torch.from_numpy(bits_values(x)), (n,),
                                           weight=torch.from_numpy(bits_values(w)), eps=eps)
        assert np.abs(y - ref.numpy()).max() <= 1e-12, (rows, n, eps)


def pin_rms_scale_invariance(lib):
    """With eps = 0, multiplying a row by 2^k leaves the result unchanged, bit
    for bit (every step scales exactly)."""
    x, w = rand_rows(4, 40, seed=8)
    y = lib.rmsnorm(x, w, 0.0)
    for k in (-3, 1, 5):
        xs = bf16_bits(bits_values(x).astype(np.float32) * np.float32(2.0 ** k))
        assert np.array_equal(lib.rmsnorm(xs, w, 0.0), y), k


def pin_rms_unit_rms(lib):
    """Gain one, eps = 0: every output row has mean square one."""
    x, _ = rand_rows(6, 100, seed=9, scale=7.0)
    ones = bf16_bits(np.ones(100, np.float32))
    y = lib.rmsnorm(x, ones, 0.0)
    assert np.abs((y ** 2).mean(axis=1) - 1.0).max() <= 1e-12


def pin_rms_constant_row(lib):
    """A row of one value c maps to c / sqrt(c^2 + eps) * w."""
    n, eps = 32, 0.5
    _, w = rand_rows(1, n, seed=10)
    for c in (0.25, -3.0, 2.0):
        x = bf16_bits(np.full((1, n), c, np.float32))
        y = lib.rmsnorm(x, w, eps)
        want = c / np.sqrt(c * c + eps) * bits_values(w)
        assert np.abs(y[0] - want).max() <= 1e-14, c


ALL_RMS_PINS = [pin_rms_mpmath, pin_rms_torch, pin_rms_scale_invariance, pin_rms_unit_rms,
                pin_rms_constant_row]
