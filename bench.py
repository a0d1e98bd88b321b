#!/usr/bin/env python3
"""Benchmark of the MI355X attention forward pass (one GPU).

A step is one call of the whole hot path -- tessera_attn_fwd on one batch of
seeded synthetic Q/K/V already resident in HBM -- on the long-context causal
GQA workload B=1, Hq=32, Hkv=8, T=16384, D=128 (bf16).  The metric is
causal-adjusted attention TFLOP/s, F = 4*B*Hq*T^2*D / 2, and its fraction of
the MI355X dense bf16 MFMA peak (2516.6 TFLOP/s = 256 CU * 4096 flop/clk *
2.4 GHz).

Printed: ONE JSON line with the metric, a roofline object for the attention
kernel (achieved from HIP events around the timed steps on the kernel's
stream), the fp64 CPU oracle timed on a bounded sample of the same workload
(the CPU baseline), a parity check of the timed output against that oracle
sample, and the secondary workloads timed the same way (each after at least
0.2 s of warm-up launches, since they follow the CPU sample's idle spell).

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME]
"""
from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import re
import sys
import time
from pathlib import Path

ROOT = Path(__file__).resolve().parent
sys.path.insert(0, str(ROOT))

PEAK_BF16_TFLOPS = 2516.6     # dense bf16 MFMA: 256 CU x 4096 flop/clk x 2.4 GHz
PEAK_HBM_GBS = 8000.0
RMS_WORKING_SET = 1 << 30     # bytes of x/y copies the RMSNorm line rotates over
HEADLINE = "t16384_d128"
# every other forward workload, each timed and checked against the oracle
SECONDARY = ["t4096_outliers", "t4096_outlier_rows", "t2048", "t2048_full",
             "chunk2048_t16384_d128", "tiny_t128", "fp32_t64"]
BACKWARD = ["t16384_d128", "t4096_outliers", "t2048"]
KERNEL_SOURCE = ROOT / "attention_flashattention_fwd_amd" / "csrc" / "tessera_attn.hip"
PROFILES = ROOT / "profiles"
# Parity bars.  Forward: bf16 max-abs 2e-2 and mean-abs 2e-3 (O and lse
# separately), fp32 max-abs 1e-4.  Backward, per tensor X: max-abs 2^-6 of
# max|X| and mean-abs 2^-8 of RMS(X), the bar derived from the rounding model
# of the bf16 pipeline in tests/bwd_rounding.py.
BF16_MAX, BF16_MEAN, F32_MAX = 2e-2, 2e-3, 1e-4
BWD_MAX, BWD_MEAN = 2.0 ** -6, 2.0 ** -8
# forward workloads whose oracle pass over every element takes about a second
EVERY_ELEMENT_FLOPS = 1e11


def parse_args(argv=None):
    p = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--gpus", type=int, default=1)
    p.add_argument("--steps", type=int, default=50)
    p.add_argument("--warmup", type=int, default=20)
    p.add_argument("--workload", default=HEADLINE)
    p.add_argument("--cpu-seconds", type=float, default=15.0,
                   help="wall-time budget of the CPU-oracle baseline sample")
    p.add_argument("--no-secondary", action="store_true", help="skip the secondary workloads")
    p.add_argument("--no-cpu", action="store_true", help="skip the CPU baseline (profiling runs)")
    p.add_argument("--backward-only", action="store_true",
                   help="only time the attention backward workload(s) (profiling runs)")
    p.add_argument("--rmsnorm-only", action="store_true",
                   help="only time the fused RMSNorm workload(s) (profiling runs)")
    p.add_argument("--paged-only", action="store_true",
                   help="only time the paged-decode workload(s) (profiling runs)")
    p.add_argument("--hbm-calibration", action="store_true",
                   help="only run a plain 1 GiB device copy (to scale HBM counters)")
    p.add_argument("--gemm-calibration", action="store_true",
                   help="only time the vendor bf16 GEMM (torch.matmul, 16384^3): the MFMA "
                        "rate a library contraction reaches on this part, for context")
    return p.parse_args(argv)


_T0 = time.perf_counter()


def progress(msg: str) -> None:
    """One line on stderr per finished phase (the JSON line stays alone on stdout)."""
    print(f"bench: {msg} ({time.perf_counter() - _T0:.0f} s)", file=sys.stderr, flush=True)


def source_digest() -> str:
    """SHA-256 prefix of the kernel source with comments and whitespace runs
    removed: a comment edit keeps the recorded counters valid, a code edit
    does not."""
    text = KERNEL_SOURCE.read_text()
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    text = " ".join(text.split())
    return hashlib.sha256(text.encode()).hexdigest()[:16]


def traffic_summary(name: str) -> Path:
    return PROFILES / f"hbm_traffic_attn_fwd_bf16_{name}.md"


def recorded_traffic(name: str):
    """HBM bytes per launch of the forward on workload `name` from the
    committed rocprofv3 counter summary, if one was taken on the current
    kernel source; else (None, None)."""
    path = traffic_summary(name)
    if not path.exists():
        return None, None
    text = path.read_text()
    m_src = re.search(r"kernel_source_sha256_16:\s*([0-9a-f]+)", text)
    m_b = re.search(r"hbm_bytes_per_launch:\s*([0-9.eE+]+)", text)
    if not m_src or not m_b or m_src.group(1) != source_digest():
        return None, None
    extra = {}
    for key in ("fetch_bytes_per_launch", "write_bytes_per_launch", "algorithmic_bytes_per_launch",
                "mfma_busy_pct", "shader_clock_ghz", "vendor_gemm_bf16_tflops"):
        m = re.search(rf"{key}:\s*([0-9.eE+]+)", text)
        if m:
            extra[key] = float(m.group(1))
    return float(m_b.group(1)), extra


class Markers:
    """roctx ranges around the bench's launch loops, so a profiler trace
    (rocprofv3 --marker-trace) shows which workload and phase a kernel belongs
    to.  Without the roctx library the ranges are skipped; nothing else
    depends on them."""

    def __init__(self):
        import ctypes
        self.lib = None
        for name in ("librocprofiler-sdk-roctx.so.1", "libroctx64.so.4"):
            try:
                lib = ctypes.CDLL(name)
                lib.roctxRangePushA.argtypes = [ctypes.c_char_p]
                lib.roctxRangePushA.restype = ctypes.c_int
                lib.roctxRangePop.argtypes = []
                lib.roctxRangePop.restype = ctypes.c_int
                self.lib = lib
                break
            except (OSError, AttributeError):
                continue

    def push(self, label: str) -> None:
        if self.lib is not None:
            self.lib.roctxRangePushA(label.encode())

    def pop(self) -> None:
        if self.lib is not None:
            self.lib.roctxRangePop()


MARKERS = None


def markers() -> Markers:
    global MARKERS
    if MARKERS is None:
        MARKERS = Markers()
    return MARKERS


def time_steps(torch, fn, steps, warmup, stream, warm_seconds=0.0, label="step"):
    """W untimed steps (continued until warm_seconds of wall time have passed:
    after an idle spell the shader clock takes tens of milliseconds of load to
    settle), then K timed steps back to back, bracketed by synchronisation and
    by two HIP events on the kernel's stream.  A second pass of K steps, with
    an event between consecutive launches, gives the per-launch median and
    minimum; it is not part of the timed region.  Each phase is a roctx range
    named after `label`."""
    mk = markers()
    with torch.cuda.stream(stream):
        mk.push(f"{label}: warm-up")
        t_w = time.perf_counter()
        n = 0
        while n < warmup or time.perf_counter() - t_w < warm_seconds:
            fn()
            n += 1
            if n % 8 == 0:
                torch.cuda.synchronize()   # keep the host clock in step with the GPU
        torch.cuda.synchronize()
        mk.pop()
        start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        mk.push(f"{label}: timed x{steps}")
        t0 = time.perf_counter()
        start.record(stream)
        for _ in range(steps):
            fn()
        end.record(stream)
        torch.cuda.synchronize()
        wall = time.perf_counter() - t0
        mk.pop()
        gpu_ms = start.elapsed_time(end) / steps
        mk.push(f"{label}: per-launch events x{steps}")
        events = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
        events[0].record(stream)
        for i in range(steps):
            fn()
            events[i + 1].record(stream)
        torch.cuda.synchronize()
        mk.pop()
    per = sorted(events[i].elapsed_time(events[i + 1]) for i in range(steps))
    return gpu_ms, wall * 1e3 / steps, per[len(per) // 2], per[0]


def cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return ""


def forward_parity(w, eo, el):
    """Parity record of forward errors eo (O) and el (lse) against the oracle."""
    rec = {"O_max_abs": float(eo.max()), "O_mean_abs": float(eo.mean()),
           "lse_max_abs": float(el.max()), "lse_mean_abs": float(el.mean())}
    if w.dtype == "fp32":
        rec["bar"] = f"max-abs {F32_MAX:g}"
        rec["ok"] = bool(eo.max() <= F32_MAX and el.max() <= F32_MAX)
    else:
        rec["bar"] = f"max-abs {BF16_MAX:g}, mean-abs {BF16_MEAN:g}"
        rec["ok"] = bool(eo.max() <= BF16_MAX and eo.mean() <= BF16_MEAN
                         and el.max() <= BF16_MAX and el.mean() <= BF16_MEAN)
    return rec


def cpu_baseline(w, q, k, v, out, lse, budget_s, every=False):
    """The fp64 oracle on the workload, timed on the host cores, checking the
    GPU's timed output on what it computes.  every=True: all rows at once
    (small workloads).  Otherwise random query rows until the time budget is
    spent.  The rate is in TFLOP/s with the same causal-adjusted count, 4*D
    per visible (query, key) pair.  A continuation workload (Tq < Tk) takes
    its rows from the full forward over the Tk positions (q holds the full
    query tensor then)."""
    import numpy as np
    import oracle
    import torch

    kv = hasattr(w, "Tk")
    Tq, Tk = (w.Tq, w.Tk) if kv else (w.T, w.T)
    qb, kb, vb = inputs_bits(q), inputs_bits(k), inputs_bits(v)
    threads = oracle.threads(0)
    if every and not kv:
        t0 = time.perf_counter()
        O_ref, l_ref = oracle.attn_fwd(qb, kb, vb, w.causal, w.scale, nthreads=threads)
        elapsed = time.perf_counter() - t0
        o = out.float().cpu().numpy().astype(np.float64)
        l = lse.cpu().numpy().astype(np.float64)
        parity = {"rows_checked": int(w.B * w.Hq * w.T), "every_element": True,
                  **forward_parity(w, np.abs(o - O_ref), np.abs(l - l_ref))}
        sample = f"every row of the workload ({w.flops / 1e9:.2f} GFLOP, {elapsed:.2f} s"
        flops = w.flops
    else:
        rng = np.random.default_rng(1234)
        total_rows = w.B * w.Hq * Tq
        batch = max(64, 16 * threads)
        flops = 0.0
        elapsed = 0.0
        rows_all, O_all, l_all = [], [], []
        while elapsed < budget_s:
            rows = rng.integers(0, total_rows, batch).astype(np.int64)
            i = rows % Tq
            full = (rows // Tq) * Tk + i + (Tk - Tq)   # the row of the full forward
            t0 = time.perf_counter()
            O, l = oracle.attn_rows(qb, kb, vb, w.causal, w.scale, full, nthreads=threads)
            elapsed += time.perf_counter() - t0
            pos = i + (Tk - Tq)
            flops += float(np.sum(4.0 * w.D * ((pos + 1) if w.causal else np.full_like(pos, Tk))))
            rows_all.append(rows)
            O_all.append(O)
            l_all.append(l)
            if len(rows_all) * batch >= total_rows:
                break
        rows = np.concatenate(rows_all)
        idx = torch.from_numpy(rows).to(out.device)
        o = out.reshape(-1, w.D)[idx].float().cpu().numpy().astype(np.float64)
        l = lse.reshape(-1)[idx].cpu().numpy().astype(np.float64)
        parity = {"rows_checked": int(len(rows)),
                  **forward_parity(w, np.abs(o - np.concatenate(O_all)),
                                   np.abs(l - np.concatenate(l_all)))}
        sample = (f"{len(rows)} random query rows of the same workload ({flops / 1e9:.1f} "
                  f"GFLOP, {elapsed:.1f} s")
    baseline = {
        "value": flops / elapsed / 1e12, "unit": "TFLOP/s", "cores": threads, "kind": "oracle",
        "sample": f"{sample}, fp64, OpenMP {threads} threads, {cpu_model()})",
    }
    return baseline, parity


def inputs_bits(t):
    from attention_flashattention_fwd_amd import inputs
    return inputs.bits(t)


def main(argv=None):
    args = parse_args(argv)
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only; --gpus {args.gpus} is not supported "
              "(the attention path here runs on one GPU; more GPUs would each take a share "
              "of the batch and KV heads in a process of their own)",
              file=sys.stderr)
        return 2

    import torch
    from attention_flashattention_fwd_amd import binding, inputs

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    stream = torch.cuda.Stream(dev)

    if args.hbm_calibration:
        n = 1 << 30
        src = torch.empty(n, dtype=torch.uint8, device=dev).fill_(1)
        dst = torch.empty_like(src)
        for _ in range(max(1, args.steps)):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"hbm_calibration_copy_bytes": n, "launches": max(1, args.steps)}))
        return 0

    if args.gemm_calibration:
        n = 16384
        g = torch.Generator(device=dev).manual_seed(0)
        a = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
        b = torch.randn(n, n, device=dev, dtype=torch.bfloat16, generator=g)
        c = torch.empty_like(a)
        gemm_ms, _, _, _ = time_steps(torch, lambda: torch.matmul(a, b, out=c),
                                      max(1, args.steps), args.warmup, stream,
                                      label="vendor gemm")
        tflops = 2.0 * n ** 3 / (gemm_ms * 1e-3) / 1e12
        print(json.dumps({"gemm_calibration": f"bf16 {n}x{n}x{n} torch.matmul",
                          "ms_per_call": round(gemm_ms, 4), "tflops": round(tflops, 1),
                          "pct_of_peak": round(100.0 * tflops / PEAK_BF16_TFLOPS, 2),
                          "launches": max(1, args.steps) + args.warmup}))
        return 0

    def rmsnorm_lines():
        """The fused RMSNorm (HBM-bound): bytes moved per call over the kernel time."""
        res = {}
        for name, rw in inputs.RMS_WORKLOADS.items():
            x, g = inputs.make_rmsnorm(rw.rows, rw.n, rw.seed)
            xd, gd = x.to(dev), g.to(dev)
            # Consecutive calls rotate over copies of x and y whose total exceeds the
            # 256 MB Infinity Cache several times over, so that each call reads x from
            # HBM, as a layer's activations larger than the caches would be: with one
            # buffer pair of 128 MB tensors, part of x stays cached between calls.
            pair_bytes = 2 * xd.numel() * 2
            npairs = max(2, min(16, -(-RMS_WORKING_SET // pair_bytes)))
            xs = [xd] + [xd.clone() for _ in range(npairs - 1)]
            ys = [torch.empty_like(xd) for _ in range(npairs)]
            yd = ys[0]
            torch.cuda.synchronize()
            turn = [0]

            def fn():
                j = turn[0] % npairs
                turn[0] += 1
                binding.rmsnorm_fwd_into(xs[j], gd, ys[j], rw.eps, stream=stream)

            r_ms, _, r_med, _ = time_steps(torch, fn, max(20, args.steps), args.warmup, stream,
                                           warm_seconds=0.2, label=f"rmsnorm {name}")
            gbs = rw.bytes / (r_ms * 1e-3) / 1e9
            # context: a plain device copy of the same tensors (torch), rotated the same way:
            # what HBM gives a read-once / write-once pass on this part

            def copy():
                j = turn[0] % npairs
                turn[0] += 1
                ys[j].copy_(xs[j])

            c_ms, _, _, _ = time_steps(torch, copy, max(20, args.steps), args.warmup, stream,
                                       warm_seconds=0.1, label="device copy")
            copy_gbs = 2.0 * xd.numel() * 2 / (c_ms * 1e-3) / 1e9
            binding.rmsnorm_fwd_into(xd, gd, yd, rw.eps, stream=stream)   # the copies overwrote y
            torch.cuda.synchronize()
            del xs[1:], ys[1:]
            # the oracle on a sample of rows (CPU baseline), which also checks them
            import numpy as np

            import oracle
            rows = np.arange(rw.rows)   # every row: the oracle takes milliseconds here
            xb, wb = inputs.bits(x), inputs.bits(g)
            t0 = time.perf_counter()
            y_ref = oracle.rmsnorm(xb[rows], wb, rw.eps)
            cpu_s = time.perf_counter() - t0
            y = yd[torch.from_numpy(rows).to(dev)].float().cpu().numpy().astype(np.float64)
            bound = (2.0 ** -8 + (rw.n / 64 + 16) * 2.0 ** -24) * np.abs(y_ref)
            worst = float(np.max(np.abs(y - y_ref) / np.maximum(bound, 1e-300)))
            progress(f"rmsnorm {name} timed and checked")
            res[name] = {
                "config": rw.describe(),
                "us_per_call": round(r_ms * 1e3, 2),
                "us_median": round(r_med * 1e3, 2),
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                             "device_copy_gbs": round(copy_gbs, 1)},
                "buffers": f"{npairs} x/y pairs rotated ({npairs * pair_bytes / 2**30:.2f} GiB)",
                "cpu_baseline": {
                    "value": round(2.0 * (2 * len(rows) * rw.n + rw.n) / cpu_s / 1e9, 3),
                    "unit": "GB/s", "cores": oracle.threads(0), "kind": "oracle",
                    "sample": (f"all {len(rows)} rows of the same workload ({cpu_s:.3f} s, "
                               f"fp64, {cpu_model()})")},
                "parity": {"rows": len(rows), "worst_error_over_bound": worst,
                           "ok": worst <= 1.0},
            }
        return res

    if args.rmsnorm_only:
        print(json.dumps(rmsnorm_lines()))
        return 0

    def backward_lines():
        """The attention backward on the long-context, T=4096 and T=2048 workloads
        (the last a grid small enough for the one-step-late dk/dv build).  Rate
        counted the usual way, 2.5x the forward's flops (the five products S,
        dP, dq, dk, dv); the two kernels here execute seven (S and dP once in
        each).  The timed output is checked against the oracle: at T=4096 the
        whole first GQA group of batch element 0 (its G query heads, all rows);
        at T=16384 random rows (query rows of any head, key rows of one KV
        head), each rebuilt from the definitions.  Bar per tensor X: max-abs
        2^-6 max|X| (max|X| of the whole GPU tensor where only rows are
        checked), mean-abs 2^-8 RMS(X) (RMS of the checked reference values)."""
        import numpy as np

        import oracle
        res = {}
        for name in BACKWARD:
            w = inputs.WORKLOADS[name]
            q, k, v = inputs.make_workload(w)
            g = torch.Generator().manual_seed(7)
            do = torch.randn(q.shape, generator=g).to(torch.bfloat16)
            qd, kd, vd, dod = (t.to(dev) for t in (q, k, v, do))
            out, lse = binding.attn_fwd(qd, kd, vd, causal=w.causal, scale=w.scale)
            fn = lambda: binding.attn_bwd(qd, kd, vd, out, lse, dod, w.causal,  # noqa: E731
                                          w.scale, stream=stream)
            b_ms, _, b_med, _ = time_steps(torch, fn, max(5, args.steps // 5), args.warmup,
                                           stream, warm_seconds=0.2, label=f"backward {name}")
            tf = 2.5 * w.flops / (b_ms * 1e-3) / 1e12
            progress(f"backward {name} timed")
            line = {
                "config": w.describe() + ", backward (dq, dk, dv)",
                "us_per_call": round(b_ms * 1e3, 2),
                "us_median": round(b_med * 1e3, 2),
                "tflops": round(tf, 1),
                "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 2),
            }
            res[f"bwd_{name}"] = line
            if args.no_cpu:
                continue
            dq, dk, dv, delta = fn()
            torch.cuda.synchronize()
            G = w.Hq // w.Hkv
            worst = 0.0

            def bar_ratio(got, ref, top, sample_ref):
                e = np.abs(got - ref)
                rms = np.sqrt(np.mean(sample_ref * sample_ref))
                return max(e.max() / (BWD_MAX * top), e.mean() / (BWD_MEAN * rms))

            if w.T <= 4096:
                sl = [inputs.bits(t[:1, :G]) for t in (q, do)]
                kv1 = [inputs.bits(t[:1, :1]) for t in (k, v)]
                t0 = time.perf_counter()
                rq, rk, rv, _ = oracle.attn_bwd(sl[0], kv1[0], kv1[1], sl[1], w.causal, w.scale)
                cpu_s = time.perf_counter() - t0
                work = 2.5 * w.flops * G / (w.B * w.Hq)
                for got, ref in ((dq[:1, :G], rq), (dk[:1, :1], rk), (dv[:1, :1], rv)):
                    gv = got.float().cpu().numpy().astype(np.float64)
                    worst = max(worst, bar_ratio(gv, ref, np.abs(ref).max(), ref))
                sample = (f"batch element 0, query heads 0..{G - 1} with KV head 0, all {w.T} "
                          f"rows ({work / 1e9:.1f} GFLOP counted as 2.5x the forward's")
                where = "b=0, KV head 0, every element"
            else:
                rng = np.random.default_rng(99)
                T = w.T
                qrows = np.sort(rng.integers(0, w.B * w.Hq * T, 64)).astype(np.int64)
                g0 = int(rng.integers(0, w.B * w.Hkv))
                krows = np.sort(g0 * T + rng.integers(0, T, 32)).astype(np.int64)
                t0 = time.perf_counter()
                rq, rd, rk, rv = oracle.attn_bwd_rows(*(inputs.bits(t) for t in (q, k, v, do)),
                                                      w.causal, w.scale, qrows, krows)
                cpu_s = time.perf_counter() - t0
                # work: the statistics of every query row of the key rows' group
                # (scores and dO.v over their visible keys), plus each row's own sums
                vis = lambda i: (i + 1) if w.causal else np.full_like(i, T)  # noqa: E731
                work = (4.0 * w.D * G * float(vis(np.arange(T)).sum())
                        + 6.0 * w.D * float(vis(qrows % T).sum())
                        + 4.0 * w.D * G * float(np.sum(T - krows % T)))
                for full, rows, ref in ((dq, qrows, rq), (delta, qrows, rd), (dk, krows, rk),
                                        (dv, krows, rv)):
                    f = full.float()
                    top = float(f.abs().max())
                    idx = torch.from_numpy(rows).to(dev)
                    gv = (f.reshape(-1, w.D)[idx] if f.dim() == 4 else f.reshape(-1)[idx])
                    worst = max(worst, bar_ratio(gv.cpu().numpy().astype(np.float64), ref, top, ref))
                sample = (f"dq, Delta of {len(qrows)} random query rows and dk, dv of "
                          f"{len(krows)} random key rows of (b, KV head) {divmod(g0, w.Hkv)}, "
                          f"each from the definitions ({work / 1e9:.1f} GFLOP")
                where = f"{len(qrows)} random query rows, {len(krows)} random key rows"
            progress(f"backward {name} oracle check done")
            line.update({
                "cpu_baseline": {
                    "value": round(work / cpu_s / 1e12, 5), "unit": "TFLOP/s",
                    "cores": oracle.threads(0), "kind": "oracle",
                    "sample": f"{sample}, {cpu_s:.1f} s, fp64, {cpu_model()})"},
                "parity": {"checked": where, "worst_error_over_bar": float(worst),
                           "bar": "max-abs 2^-6 max|X|, mean-abs 2^-8 RMS(X)",
                           "ok": bool(worst <= 1.0)},
            })
        return res

    if args.backward_only:
        print(json.dumps(backward_lines()))
        return 0

    def paged_lines():
        """Decode over the block-paged cache (HBM-bound): the bytes one call must
        move (every cached K/V row once, q, out, lse, table entries) over the
        time of the call (split kernel plus merge kernel).  Four sequences of the
        timed output, the longest among them, are checked against the oracle."""
        import numpy as np

        import oracle

        res = {}
        for name, pw in inputs.PAGED_WORKLOADS.items():
            q, kc, vc, table, cl = inputs.make_paged_workload(pw)
            qd, kd, vd, td, cd = (t.to(dev) for t in (q, kc, vc, table, cl))
            out = torch.empty_like(qd)
            lse = torch.empty(qd.shape[:3], dtype=torch.float32, device=dev)
            nws = binding.paged_workspace_bytes(pw.B, pw.Hq, pw.Hkv, pw.Tq, pw.D, pw.block_size,
                                                pw.max_blocks)
            ws = torch.empty(max(nws, 1), dtype=torch.uint8, device=dev) if nws else None
            torch.cuda.synchronize()
            fn = lambda: binding.paged_decode_into(qd, kd, vd, td, cd, out, lse, ws,  # noqa: E731
                                                   pw.causal, pw.scale, stream=stream)
            p_ms, _, p_med, p_min = time_steps(torch, fn, max(20, args.steps), args.warmup,
                                               stream, warm_seconds=0.2,
                                               label=f"paged decode {name}")
            nbytes = inputs.paged_bytes(cl.numpy(), pw.Hq, pw.Hkv, pw.Tq, pw.D, pw.block_size)
            gbs = nbytes / (p_ms * 1e-3) / 1e9
            n = cl.numpy()
            pick = np.array(sorted({int(n.argmax()), 0, pw.B // 2, pw.B - 1}))
            t0 = time.perf_counter()
            O_ref, l_ref = oracle.paged_decode(inputs.bits(q[pick]), inputs.bits(kc),
                                               inputs.bits(vc), table.numpy()[pick], n[pick],
                                               pw.causal, pw.scale)
            cpu_s = time.perf_counter() - t0
            cpu_bytes = inputs.paged_bytes(n[pick], pw.Hq, pw.Hkv, pw.Tq, pw.D, pw.block_size)
            o = out[torch.from_numpy(pick).to(dev)].float().cpu().numpy()
            lg = lse[torch.from_numpy(pick).to(dev)].cpu().numpy()
            eo, el = float(np.abs(o - O_ref).max()), float(np.abs(lg - l_ref).max())
            progress(f"paged decode {name} timed and checked")
            res[name] = {
                "config": pw.describe(),
                "tokens_cached": int(n.sum()),
                "bytes_per_call": nbytes,
                "us_per_call": round(p_ms * 1e3, 2),
                "us_median": round(p_med * 1e3, 2),
                "us_min": round(p_min * 1e3, 2),
                "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": PEAK_HBM_GBS,
                             "unit": "GB/s", "frac": round(gbs / PEAK_HBM_GBS, 4),
                             "kernel": f"paged_decode_kernel<{pw.D}> + paged_combine_kernel"},
                "cpu_baseline": {
                    "value": round(cpu_bytes / cpu_s / 1e9, 3), "unit": "GB/s",
                    "cores": oracle.threads(0), "kind": "oracle",
                    "sample": (f"sequences {pick.tolist()} of the same batch "
                               f"({int(n[pick].sum())} cached tokens, {cpu_s:.2f} s, fp64, "
                               f"{cpu_model()})")},
                "parity": {"sequences": pick.tolist(), "max_abs_err_O": eo,
                           "max_abs_err_lse": el, "ok": eo <= 2e-2 and el <= 2e-2},
            }
        return res

    if args.paged_only:
        print(json.dumps(paged_lines()))
        return 0

    def measure(name, steps, warmup, cpu_seconds, warm_seconds=0.0):
        """Time the forward on workload `name`; with cpu_seconds set (not None),
        also check the timed output against the oracle and time the oracle
        (every element for the small workloads, else random rows for about
        cpu_seconds)."""
        if name in inputs.KV_WORKLOADS:   # Tq new rows against Tk cached rows
            w = inputs.KV_WORKLOADS[name]
            q, k, v = inputs.make_kv_workload(w, full_q=True)
            qd = q[:, :, w.Tk - w.Tq:].contiguous().to(dev)
            kd, vd = k.to(dev), v.to(dev)
            out = torch.empty_like(qd)
            lse = torch.empty((w.B, w.Hq, w.Tq), dtype=torch.float32, device=dev)
            fn = lambda: binding.attn_fwd_kv_into(qd, kd, vd, out, lse,  # noqa: E731
                                                  w.causal, w.scale, stream=stream)
        else:
            w = inputs.WORKLOADS[name]
            q, k, v = inputs.make_workload(w)
            qd, kd, vd = (t.to(dev) for t in (q, k, v))
            out = torch.empty_like(qd)
            lse = torch.empty((w.B, w.Hq, w.T), dtype=torch.float32, device=dev)
            fn = lambda: binding.attn_fwd_into(qd, kd, vd, out, lse,  # noqa: E731
                                               w.causal, w.scale, stream=stream)
        torch.cuda.synchronize()
        gpu_ms, wall_ms, med_ms, min_ms = time_steps(torch, fn, steps, warmup, stream,
                                                     warm_seconds, label=f"forward {name}")
        res = {"w": w, "gpu_ms": gpu_ms, "wall_ms": wall_ms, "med_ms": med_ms, "min_ms": min_ms}
        progress(f"forward {name} timed")
        if cpu_seconds is not None:
            every = w.flops <= EVERY_ELEMENT_FLOPS and not hasattr(w, "Tk")
            res["cpu"], res["parity"] = cpu_baseline(w, q, k, v, out, lse, cpu_seconds, every)
            progress(f"forward {name}: oracle baseline and parity done "
                     f"(ok={res['parity']['ok']})")
        return res

    if args.workload not in inputs.WORKLOADS and args.workload not in inputs.KV_WORKLOADS:
        print(f"unknown workload {args.workload!r}", file=sys.stderr)
        return 2
    head = measure(args.workload, args.steps, args.warmup,
                   None if args.no_cpu else args.cpu_seconds)
    w = head["w"]
    tflops = w.flops / (head["wall_ms"] * 1e-3) / 1e12
    achieved = w.flops / (head["gpu_ms"] * 1e-3) / 1e12
    traffic, counters = recorded_traffic(w.name)
    failed = []
    if "parity" in head and not head["parity"]["ok"]:
        failed.append(w.name)

    secondary = {}
    if not args.no_secondary:
        for name in SECONDARY:
            if name == w.name:
                continue
            r = measure(name, max(5, args.steps // 2), args.warmup,
                        None if args.no_cpu else min(3.0, args.cpu_seconds), warm_seconds=0.2)
            rw = r["w"]
            tf = rw.flops / (r["gpu_ms"] * 1e-3) / 1e12
            sec = {
                "config": rw.describe(),
                "us_per_call": round(r["gpu_ms"] * 1e3, 2),
                "us_median": round(r["med_ms"] * 1e3, 2),
                "tflops": round(tf, 3 if tf < 10 else 1),
                "pct_of_peak": round(100 * tf / PEAK_BF16_TFLOPS, 3),
            }
            if rw.dtype == "fp32":
                sec["note"] = ("fp32 inputs run on the vector ALUs (fp32 peak 157.3 TFLOP/s); "
                               "the bf16 peak fraction is context only")
            s_traffic, s_counters = recorded_traffic(name)
            if s_traffic is not None:
                sec["traffic"] = s_traffic
                sec["hbm_gbs"] = round(s_traffic / (r["gpu_ms"] * 1e-3) / 1e9, 1)
                sec["counters"] = s_counters
            if "parity" in r:
                sec["cpu_baseline"] = r["cpu"]
                sec["parity"] = r["parity"]
                if not r["parity"]["ok"]:
                    failed.append(name)
            secondary[name] = sec

    if not args.no_secondary:
        for extra in (rmsnorm_lines(), backward_lines(), paged_lines()):
            for name, rec in extra.items():
                if isinstance(rec.get("parity"), dict) and rec["parity"].get("ok") is False:
                    failed.append(name)
            secondary.update(extra)

    line = {
        "metric": "attention fwd TFLOP/s (causal-adjusted) and % of MI355X bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(head["wall_ms"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": w.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, bf16)",
        "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "config": {"workload": w.name, "B": w.B, "Hq": w.Hq, "Hkv": w.Hkv,
                   **({"T": w.T} if hasattr(w, "T") else {"Tq": w.Tq, "Tk": w.Tk}), "D": w.D,
                   "causal": w.causal, "scale": w.scale, "flops_per_step": w.flops,
                   "pair_exact_flops_per_step": getattr(w, "pair_flops", w.flops),
                   "parallelism": "single GPU"},
        "roofline": {
            "bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS,
            "unit": "TFLOP/s", "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
            "traffic": traffic,
            "kernel": f"attn_fwd_bf16_kernel<{w.D}>",
            "kernel_us_per_launch": round(head["gpu_ms"] * 1e3, 2),
            "kernel_us_median": round(head["med_ms"] * 1e3, 2),
            "kernel_us_min": round(head["min_ms"] * 1e3, 2),
        },
    }
    if counters:
        line["roofline"]["counters"] = counters
        line["roofline"]["hbm_gbs"] = round(traffic / (head["gpu_ms"] * 1e-3) / 1e9, 1)
        if "shader_clock_ghz" in counters:
            # the same 4096 flop/clk/CU at the clock the profiled run measured
            at_clock = 256 * 4096 * counters["shader_clock_ghz"] * 1e9 / 1e12
            line["roofline"]["frac_at_measured_clock"] = round(achieved / at_clock, 4)
        if "vendor_gemm_bf16_tflops" in counters:
            line["roofline"]["frac_of_vendor_gemm"] = round(
                achieved / counters["vendor_gemm_bf16_tflops"], 4)
    if "cpu" in head:
        line["cpu_baseline"] = head["cpu"]
        line["parity"] = head["parity"]
    if secondary:
        line["secondary"] = secondary
    line["context"] = ("the pages' only figures measure a torch reference path on an Apple M2 Pro "
                       "(~100k tok/s model forward, tessera-tiny B=2 T=128; ~200 tok/s engine "
                       "decode, 6 requests x 48 tokens): a different metric, quoted as context only")
    print(json.dumps(line))
    if failed:
        print(f"bench: parity check against the oracle FAILED for {', '.join(failed)}",
              file=sys.stderr)
        return 1
    return 0


if __name__ == "__main__":
    sys.exit(main())
