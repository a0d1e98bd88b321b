"""GPU parity of the fused RMSNorm (tessera_rmsnorm_fwd through the binding)
against the fp64 oracle.

Each output is one fp32 value rounded once to bf16, so the bar is the rounding
bound itself, element by element: |y - y_ref| <= (2^-8 + (n/64 + 16) 2^-24) |y_ref|.
Rounding to nearest with 8 significant bits is off by at most half an ulp,
2^-8 of the value just above a power of two.  The fp32 part: each lane adds
n/64 squares in sequence and the wave adds 64 partial sums in six steps
(worst case (n/64 + 6) 2^-24 relative on the mean of squares, half of that
on its inverse square root); square root, reciprocal and two products add a
few more units of 2^-24.  (n/64 + 16) 2^-24 covers both.
"""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from attention_flashattention_fwd_amd import binding, inputs
from tests.test_gpu_parity import say

pytestmark = pytest.mark.gpu


def draw(rows, n, seed, scale=1.0):
    return inputs.make_rmsnorm(rows, n, seed, scale)


def check(y_gpu: torch.Tensor, y_ref: np.ndarray, what=""):
    y = y_gpu.float().cpu().numpy().astype(np.float64)
    assert np.isfinite(y).all(), what
    n = y_ref.shape[-1]
    err = np.abs(y - y_ref)
    bound = (2.0 ** -8 + (n / 64 + 16) * 2.0 ** -24) * np.abs(y_ref) + 1e-30
    worst = (err / bound).max()
    say(f"{what} max-abs {err.max():.3e}  worst err/bound {worst:.3f}")
    assert worst <= 1.0, what


CASES = [(1, 8), (3, 64), (7, 256), (5, 504), (100, 4096), (33, 8192),   # rows held in registers
         (9, 8200), (4, 65536),                                          # rows read twice
         (20000, 128)]                                                   # waves stride over rows


@pytest.mark.parametrize("rows,n", CASES)
@pytest.mark.parametrize("eps", [1e-6, 0.0])
def test_rmsnorm_shapes(rows, n, eps):
    x, w = draw(rows, n, seed=rows + n)
    say(f"case rmsnorm rows={rows} n={n} eps={eps}")
    y = binding.rmsnorm_fwd(x.cuda(), w.cuda(), eps)
    torch.cuda.synchronize()
    check(y, oracle.rmsnorm(inputs.bits(x), inputs.bits(w), float(np.float32(eps))),
          f"rows={rows} n={n}")


@pytest.mark.parametrize("scale", [1e-3, 100.0])
def test_rmsnorm_row_magnitudes(scale):
    x, w = draw(64, 1024, seed=5, scale=scale)
    say(f"case rmsnorm magnitude {scale}")
    y = binding.rmsnorm_fwd(x.cuda(), w.cuda(), 1e-6)
    torch.cuda.synchronize()
    check(y, oracle.rmsnorm(inputs.bits(x), inputs.bits(w), float(np.float32(1e-6))),
          f"scale={scale}")


def test_rmsnorm_in_place_and_large_eps():
    for n in (2048, 16384):
        x, w = draw(50, n, seed=n)
        ref = oracle.rmsnorm(inputs.bits(x), inputs.bits(w), 0.5)
        xd = x.cuda()
        binding.rmsnorm_fwd_into(xd, w.cuda(), xd, 0.5)
        torch.cuda.synchronize()
        check(xd, ref, f"in place n={n}")


def test_rmsnorm_leading_dims_and_argument_checks():
    x, w = draw(6, 512, seed=2)
    y = binding.rmsnorm_fwd(x.view(2, 3, 512).cuda(), w.cuda())
    torch.cuda.synchronize()
    check(y.view(6, 512), oracle.rmsnorm(inputs.bits(x), inputs.bits(w), float(np.float32(1e-6))),
          "3-D input")
    with pytest.raises(RuntimeError, match="eps"):
        binding.rmsnorm_fwd(x.cuda(), w.cuda(), -1.0)
    with pytest.raises(ValueError):
        binding.rmsnorm_fwd(x.cuda().float(), w.cuda())


@pytest.mark.parametrize("name", sorted(inputs.RMS_WORKLOADS))
def test_rmsnorm_benchmarked_workload(name):
    """The benchmarked size, every element against the oracle."""
    wl = inputs.RMS_WORKLOADS[name]
    x, w = inputs.make_rmsnorm(wl.rows, wl.n, wl.seed)
    say(f"workload {name}: {wl.describe()}")
    y = binding.rmsnorm_fwd(x.cuda(), w.cuda(), wl.eps)
    torch.cuda.synchronize()
    check(y, oracle.rmsnorm(inputs.bits(x), inputs.bits(w), float(np.float32(wl.eps))), name)


def test_rmsnorm_offsets_past_int32():
    """x and y of (2^19 + 8) x 4096 elements (more than 2^31): the last eight
    rows start past 2^31 elements.  Those, the first and the row just before
    the boundary are checked against the oracle."""
    rows, n, eps = 2 ** 19 + 8, 4096, 1e-6
    assert rows * n > 2 ** 31 and (2 ** 19) * n == 2 ** 31
    dev = torch.device("cuda:0")
    say(f"case rmsnorm int32-overflowing offsets rows={rows} n={n}")
    x, w = inputs.randn_on_device(((rows, n), (n,)), seed=25, device=dev)
    y = binding.rmsnorm_fwd(x, w, eps)
    torch.cuda.synchronize()
    pick = torch.tensor([0, 2 ** 19 - 1] + list(range(2 ** 19, rows)), device=dev)
    xs, ys = x[pick].cpu(), y[pick]
    check(ys, oracle.rmsnorm(inputs.bits(xs), inputs.bits(w.cpu()), float(np.float32(eps))),
          "rows past 2^31 elements")
    del x, y
    torch.cuda.empty_cache()
