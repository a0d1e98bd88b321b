"""Per-phase cycle accounting of the bf16 forward kernel (a profiling tool).

Builds an instrumented copy of csrc/tessera_attn.hip (the same kernels, plus
timestamps) into attention_flashattention_fwd_amd/libtessera_attn_probe.so,
then runs it on forward workloads and reports, from the GPU's own clocks:

  * per work item: its XCD, compute unit, start and end (s_memrealtime,
    100 MHz) and number of key tiles;
  * per wave, summed over the steady-state tiles (the first two and the last
    two of an item are left out): the shader-clock cycles (s_memtime) of its
    MFMA phases and of its vector (softmax) phases, separately for the
    leading and the lagging wave of each SIMD;
  * per XCD: the last end, the earliest CU end and microseconds per tile, which
    show how evenly the dies share the work; per compute unit: its items, key
    tiles and last end;
  * a least-squares fit of item duration = fixed part + tiles x per-tile part
    (the fixed part is what an item's start and end cost), and the spread of
    the items' starts and ends over the launch.

The instrumentation adds only timestamp reads and one store per wave at the
start and end of each item; the timed launch rate of the instrumented build
is printed next to the library's own.

    python -m attention_flashattention_fwd_amd.phase_probe --build        (CPU; hipcc)
    python -m attention_flashattention_fwd_amd.phase_probe [workload ...]  (GPU)
"""
from __future__ import annotations

import argparse
import ctypes
import json
import subprocess
import sys
import tempfile
import time
from pathlib import Path

import numpy as np

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
SOURCE = PKG / "csrc" / "tessera_attn.hip"
PROBE_LIB = PKG / "libtessera_attn_probe.so"
WORDS = 10   # per (item, wave) record

# (anchor, replacement) pairs applied to the kernel source, in order.
PATCHES = [
    ("    uint32_t *queue;   // work queues of a persistent launch, or null (one item per workgroup)\n",
     "    uint32_t *queue;   // work queues of a persistent launch, or null (one item per workgroup)\n"
     "    uint32_t *probe;   // timestamp records (instrumented build)\n"),
    ("    const bool causal = a.causal != 0;\n",
     "    const bool causal = a.causal != 0;\n"
     "    uint32_t pm = 0, pv = 0, pt = 0, ta = 0;\n"
     "    if (a.probe && (threadIdx.x & 63) == 0) {\n"
     "        const uint64_t rt0 = __builtin_amdgcn_s_memrealtime();\n"
     "        uint32_t *p = a.probe + ((size_t)item * kWaves + (threadIdx.x >> 6)) * 10;\n"
     "        p[0] = __builtin_amdgcn_s_getreg(4 | (0 << 6) | (31 << 11));\n"
     "        p[1] = (uint32_t)rt0;\n"
     "        p[2] = (uint32_t)(rt0 >> 32);\n"
     "        p[8] = __builtin_amdgcn_s_getreg(20 | (0 << 6) | (15 << 11));\n"
     "    }\n"),
    ("    auto finish = [&](int t, int kn, int vn, bool first) __attribute__((always_inline)) {\n"
     "        phase_barrier();",
     "    auto finish = [&](int t, int kn, int vn, bool first) __attribute__((always_inline)) {\n"
     "        const uint32_t tb_ = (uint32_t)__builtin_amdgcn_s_memtime();\n"
     "        phase_barrier();\n"
     "        const uint32_t tc_ = (uint32_t)__builtin_amdgcn_s_memtime();"),
    ("            else preload<D, 2>(nullptr, vn * kTB, off, ring);\n        }\n"
     "        phase_barrier();\n    };",
     "            else preload<D, 2>(nullptr, vn * kTB, off, ring);\n        }\n"
     "        const uint32_t td_ = (uint32_t)__builtin_amdgcn_s_memtime();\n"
     "        phase_barrier();\n"
     "        if (t >= 2 && t + 2 < ntiles) { pm += tb_ - ta; pv += td_ - tc_; pt += 1; }\n    };"),
    ("        if constexpr (PAIRED) __builtin_amdgcn_s_setprio(1);\n        mfma_phase<D, 0, NQ>",
     "        ta = (uint32_t)__builtin_amdgcn_s_memtime();\n"
     "        if constexpr (PAIRED) __builtin_amdgcn_s_setprio(1);\n        mfma_phase<D, 0, NQ>"),
    ("    if (!lag) phase_barrier();\n"
     "    // The clamped loads of the last phases must land before the workgroup's\n"
     "    // LDS is released.\n"
     "    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)\n",
     "    if (!lag) phase_barrier();\n"
     "    __builtin_amdgcn_s_waitcnt(0x0F70);   // vmcnt(0)\n"
     "    {\n"
     "        const uint64_t rt1 = __builtin_amdgcn_s_memrealtime();\n"
     "        if (a.probe && lane_id_opaque() == 0) {\n"
     "            uint32_t *p = a.probe + ((size_t)item * kWaves + w) * 10;\n"
     "            p[3] = (uint32_t)rt1;\n"
     "            p[4] = (uint32_t)(rt1 >> 32);\n"
     "            p[5] = pm;\n"
     "            p[7] = pv;\n"
     "            p[9] = pt | ((uint32_t)ntiles << 16);\n"
     "        }\n"
     "    }\n"),
    ("                const tessera_attn_tile_config &c, void *stream) {\n    Bf16Args a;\n",
     "                const tessera_attn_tile_config &c, void *stream) {\n    Bf16Args a;\n"
     "    a.probe = g_probe;\n"),
    ("// Launches the bf16 build <D, RAGGED, PAIRED, NQ> over `items` work items: as",
     "uint32_t *g_probe = nullptr;\n\n"
     "// Launches the bf16 build <D, RAGGED, PAIRED, NQ> over `items` work items: as"),
]
TAIL = '\nextern "C" void tessera_probe_set(uint32_t *p) { g_probe = p; }\n'


def instrumented_source(text: str) -> str:
    for old, new in PATCHES:
        if text.count(old) != 1:
            raise RuntimeError(f"phase_probe: anchor not found once in {SOURCE.name}: {old[:60]!r}")
        text = text.replace(old, new)
    return text + TAIL


def build(verbose: bool = True) -> Path:
    from attention_flashattention_fwd_amd import build as lib_build

    with tempfile.TemporaryDirectory() as tmp:
        src = Path(tmp) / "tessera_attn_probe.hip"
        src.write_text(instrumented_source(SOURCE.read_text()))
        cmd = [lib_build.hipcc(), *lib_build.HIPCC_FLAGS, f"-I{lib_build.INCLUDE}",
               f"-I{PKG / 'csrc'}", str(src), "-o", str(PROBE_LIB)]
        res = subprocess.run(cmd, capture_output=True, text=True)
        if res.returncode != 0:
            raise RuntimeError(res.stderr[-4000:])
    if verbose:
        print(f"built {PROBE_LIB}")
    return PROBE_LIB


def analyse(rec: np.ndarray, items: int) -> dict:
    """Summary of the (item, wave, word) records of one launch."""
    r = rec.astype(np.int64) & 0xFFFFFFFF
    hw = r[:, 0, 0]
    xcc = r[:, 0, 8] & 0xF
    cu = (hw >> 8) & 0xF
    se_sh = ((hw >> 13) & 7) * 2 + ((hw >> 12) & 1)
    start = (r[:, :, 1] | (r[:, :, 2] << 32)).min(1)
    end = (r[:, :, 3] | (r[:, :, 4] << 32)).max(1)
    tiles = (r[:, 0, 9] >> 16).astype(np.int64)
    pm, pv, pt = r[:, :, 5], r[:, :, 7], r[:, :, 9] & 0xFFFF
    t0 = start.min()
    out = {"items": int(items), "span_us": float((end.max() - t0) / 100.0)}
    for name, sl in (("leading", slice(0, 4)), ("lagging", slice(4, 8))):
        n = pt[:, sl].sum()
        out[f"{name}_mfma_phase_cycles_per_tile"] = float(pm[:, sl].sum() / max(n, 1))
        out[f"{name}_vector_phase_cycles_per_tile"] = float(pv[:, sl].sum() / max(n, 1))
    per_xcd = []
    for x in range(8):
        s = xcc == x
        if not s.any():
            continue
        keys = se_sh[s] * 16 + cu[s]
        ends = [float((end[s][keys == k].max() - t0) / 100.0) for k in np.unique(keys)]
        dur = (end[s] - start[s]) / 100.0
        per_xcd.append({"xcd": x, "items": int(s.sum()), "cus": int(len(ends)),
                        "last_end_us": max(ends), "first_cu_end_us": min(ends),
                        "us_per_tile": float(np.median(dur / np.maximum(tiles[s], 1)))})
    out["per_xcd"] = per_xcd
    # per compute unit: how many items and key tiles it ran, and when its last
    # item ended (shows how evenly a grid's workgroups share the CUs)
    key_all = xcc * 256 + se_sh * 16 + cu
    cus = np.unique(key_all)
    cu_tiles = np.array([tiles[key_all == k].sum() for k in cus])
    cu_items = np.array([(key_all == k).sum() for k in cus])
    cu_end = np.array([(end[key_all == k].max() - t0) / 100.0 for k in cus])
    out["cus"] = int(len(cus))
    out["items_per_cu_min_max"] = [int(cu_items.min()), int(cu_items.max())]
    out["tiles_per_cu_min_median_max"] = [int(cu_tiles.min()), float(np.median(cu_tiles)),
                                          int(cu_tiles.max())]
    out["cu_last_end_us_min_median_max"] = [float(cu_end.min()), float(np.median(cu_end)),
                                            float(cu_end.max())]
    # item duration = fixed part + per-tile part (least squares over the items):
    # the fixed part is an item's start (Q, the first K/V tiles) and end
    dur_us = (end - start) / 100.0
    fit = np.linalg.lstsq(np.vstack([np.ones(len(tiles)), tiles]).T.astype(float), dur_us,
                          rcond=None)[0]
    out["item_fixed_us"] = float(fit[0])
    out["item_us_per_tile"] = float(fit[1])
    out["start_us_quantiles"] = [float(np.percentile((start - t0) / 100.0, q))
                                 for q in (10, 50, 90, 100)]
    out["end_us_quantiles"] = [float(np.percentile((end - t0) / 100.0, q))
                               for q in (10, 50, 90, 100)]
    return out


def run(names, repeats: int = 20) -> dict:
    import torch

    sys.path.insert(0, str(ROOT))
    from attention_flashattention_fwd_amd import binding, inputs

    L = ctypes.CDLL(str(PROBE_LIB))
    vp, i, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    L.tessera_attn_fwd.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, f, vp]
    L.tessera_attn_fwd.restype = i
    L.tessera_probe_set.argtypes = [vp]
    dev = torch.device("cuda:0")
    report = {}
    for name in names:
        w = inputs.WORKLOADS[name]
        g = torch.Generator(device=dev)
        g.manual_seed(0)
        q = torch.randn((w.B, w.Hq, w.T, w.D), generator=g, device=dev, dtype=torch.bfloat16)
        k = torch.randn((w.B, w.Hkv, w.T, w.D), generator=g, device=dev, dtype=torch.bfloat16)
        v = torch.randn((w.B, w.Hkv, w.T, w.D), generator=g, device=dev, dtype=torch.bfloat16)
        out = torch.empty_like(q)
        lse = torch.empty((w.B, w.Hq, w.T), dtype=torch.float32, device=dev)
        cfg = binding.tile_config(w.B, w.Hq, w.Hkv, w.T, w.T, w.D, int(w.causal))
        hg, rows = cfg.heads_per_workgroup, cfg.query_rows_per_wave
        items = -(-w.T // (rows * 8 // hg)) * w.B * w.Hkv * (w.Hq // w.Hkv // hg)
        buf = torch.zeros(items * 8 * WORDS, dtype=torch.int32, device=dev)
        s = torch.cuda.current_stream()

        def call(lib):
            if lib is None:
                binding.attn_fwd_into(q, k, v, out, lse, w.causal, w.scale)
            else:
                rc = lib.tessera_attn_fwd(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                          lse.data_ptr(), w.B, w.Hq, w.Hkv, w.T, w.D,
                                          int(w.causal), w.scale, s.cuda_stream)
                assert rc == 0, rc

        times = {}
        for label, lib, probe in (("library", None, None), ("instrumented", L, buf)):
            L.tessera_probe_set(buf.data_ptr() if probe is not None else None)
            t_end = time.perf_counter() + 0.3
            while time.perf_counter() < t_end:
                call(lib)
                torch.cuda.synchronize()
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record()
            for _ in range(repeats):
                call(lib)
            ev[1].record()
            torch.cuda.synchronize()
            times[label] = ev[0].elapsed_time(ev[1]) * 1e3 / repeats
        L.tessera_probe_set(None)
        rec = buf.cpu().numpy().reshape(items, 8, WORDS)
        summary = analyse(rec, items)
        summary.update({"workload": w.describe(), "config": list(cfg.as_tuple()),
                        "library_us_per_launch": times["library"],
                        "instrumented_us_per_launch": times["instrumented"]})
        report[name] = summary
        print(json.dumps({name: summary}), flush=True)
    return report


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__,
                                formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("workloads", nargs="*",
                   default=["t16384_d128", "t4096_outliers", "t2048", "t2048_full"])
    p.add_argument("--build", action="store_true", help="build the instrumented library only")
    p.add_argument("--out", default="phase_probe.json", help="JSON report (default: ./phase_probe.json)")
    args = p.parse_args(argv)
    if args.build:
        build()
        return 0
    if not PROBE_LIB.exists():
        print(f"{PROBE_LIB} is missing: run with --build first", file=sys.stderr)
        return 2
    report = run(args.workloads)
    Path(args.out).parent.mkdir(parents=True, exist_ok=True)
    Path(args.out).write_text(json.dumps(report, indent=1))
    return 0


if __name__ == "__main__":
    sys.exit(main())
