"""Offline sweep of the bf16 forward's tile configurations (the kernel set's
"autotuned tile sizes", page "Tessera: a from-scratch distillation and
serving stack in one repository", section "The kernel set and its torch
fallback").

For each head size D in {32, 64, 128}, causal or not, and each problem-size
class of the library's table (small / large: fewer or at least 1024 query
rows per compute unit), every configuration the sizes allow is timed through
tessera_attn_fwd_with_config on one benchmark shape:

    heads_per_workgroup  1, 2, 4
    query_rows_per_wave  32, 64 (D <= 64)
    workgroups_per_cu    1, 2 (D <= 64, 32 rows per wave, not persistent)
    persistent           0, 1

Each timed output is checked against the fp64 oracle on sampled rows (every
configuration must compute the same result up to rounding).  The fastest
configuration of each class becomes its rule.  Writes

    <out>/tile_sweep_attn_fwd_bf16.md   every timing, the winners marked
    <out>/tile_table.inc                the rules, in the form the library
                                        compiles (csrc/tile_table.inc)

    python -m attention_flashattention_fwd_amd.autotune [--out DIR] [--repeats N]

Needs a GPU; the library is not rebuilt (copy tile_table.inc into csrc/ and
build to adopt a new table).
"""
from __future__ import annotations

import argparse
import itertools
import re
import sys
import time
from pathlib import Path

import numpy as np

PKG = Path(__file__).resolve().parent
ROOT = PKG.parent
PEAK_BF16_TFLOPS = 2516.6
KEY_TILE = 64
LARGE_ROWS_PER_CU = 1024   # the table's class boundary (kLargeRowsPerCu in the library)

# (D, large) -> (B, Hq, Hkv, T): the benchmark workloads where they exist.
SHAPES = {
    (128, 1): (1, 32, 8, 16384),   # the long-context workload
    (128, 0): (8, 8, 2, 2048),
    (64, 1): (16, 16, 4, 4096),    # the T=4096 workload's shape
    (64, 0): (8, 8, 2, 2048),      # the T=2048 workload
    (32, 1): (16, 16, 4, 4096),
    (32, 0): (8, 8, 2, 2048),
}


def allowed(cfg, G, T, D) -> bool:
    """The rules of tessera_attn_fwd_with_config (include/tessera_attn.h)."""
    hg, rows, wg, persist = cfg
    if G % hg:
        return False
    if rows == 64 and (D > 64 or wg == 2):
        return False
    if wg == 2 and (D > 64 or T % KEY_TILE or persist):
        return False
    return True


def configs(G, T, D):
    return [c for c in itertools.product((4, 2, 1), (32, 64), (1, 2), (1, 0)) if allowed(c, G, T, D)]


def flops(B, Hq, T, D, causal) -> float:
    f = 4.0 * B * Hq * T * T * D
    return f / 2 if causal else f


def time_config(torch, binding, tensors, shape, D, causal, cfg, repeats, stream):
    """Median per-launch microseconds over `repeats` batches (HIP events on
    the launch stream) after 0.15 s of warm-up launches."""
    q, k, v, out, lse = tensors
    B, Hq, Hkv, T = shape
    tc = binding.TileConfig(*cfg)
    fn = lambda: binding.attn_fwd_with_config_into(q, k, v, out, lse, tc, causal,  # noqa: E731
                                                   stream=stream)
    with torch.cuda.stream(stream):
        t0 = time.perf_counter()
        n = 0
        while time.perf_counter() - t0 < 0.15 or n < 3:
            fn()
            n += 1
            if n % 4 == 0:
                torch.cuda.synchronize()
        torch.cuda.synchronize()
        per = max(5, min(50, int(0.05 / max((time.perf_counter() - t0) / n, 1e-6))))
        meds = []
        for _ in range(repeats):
            ev = [torch.cuda.Event(enable_timing=True) for _ in range(2)]
            ev[0].record(stream)
            for _ in range(per):
                fn()
            ev[1].record(stream)
            torch.cuda.synchronize()
            meds.append(ev[0].elapsed_time(ev[1]) * 1e3 / per)
    return float(np.median(meds))


def check_rows(torch, out, lse, D, ref):
    """Max-abs error of O and lse on the sampled rows against the oracle."""
    O_ref, l_ref, rows = ref
    idx = torch.from_numpy(rows).to(out.device)
    o = out.reshape(-1, D)[idx].float().cpu().numpy().astype(np.float64)
    l = lse.reshape(-1)[idx].cpu().numpy().astype(np.float64)
    return float(np.abs(o - O_ref).max()), float(np.abs(l - l_ref).max())


def main(argv=None) -> int:
    p = argparse.ArgumentParser(description=__doc__,
                                formatter_class=argparse.RawDescriptionHelpFormatter)
    p.add_argument("--out", default="tile_sweep_out",
                   help="folder for the table and the report (default: ./tile_sweep_out)")
    p.add_argument("--repeats", type=int, default=5)
    args = p.parse_args(argv)

    import torch

    sys.path.insert(0, str(ROOT))
    import oracle
    from attention_flashattention_fwd_amd import binding, inputs

    if not torch.cuda.is_available():
        print("autotune needs a GPU", file=sys.stderr)
        return 2
    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(dev)
    props = torch.cuda.get_device_properties(dev)
    cus = props.multi_processor_count
    out_dir = Path(args.out)
    out_dir.mkdir(parents=True, exist_ok=True)

    results = {}   # (D, causal, large) -> list of (cfg, us, err_o, err_l)
    rules = []
    for (D, large), shape in SHAPES.items():
        B, Hq, Hkv, T = shape
        assert (B * Hq * T // cus >= LARGE_ROWS_PER_CU) == bool(large), (shape, cus)
        G = Hq // Hkv
        g = torch.Generator(device=dev)
        g.manual_seed(D + 7 * large)
        q = torch.randn((B, Hq, T, D), generator=g, device=dev, dtype=torch.bfloat16)
        k = torch.randn((B, Hkv, T, D), generator=g, device=dev, dtype=torch.bfloat16)
        v = torch.randn((B, Hkv, T, D), generator=g, device=dev, dtype=torch.bfloat16)
        out = torch.empty_like(q)
        lse = torch.empty((B, Hq, T), dtype=torch.float32, device=dev)
        scale = inputs.default_scale(D)
        rng = np.random.default_rng(D)
        rows = np.unique(rng.integers(0, B * Hq * T, 48)).astype(np.int64)
        qh, kh, vh = (inputs.bits(t.cpu()) for t in (q, k, v))
        for causal in (1, 0):
            O_ref, l_ref = oracle.attn_rows(qh, kh, vh, bool(causal), scale, rows)
            ref = (O_ref, l_ref, rows)
            f = flops(B, Hq, T, D, causal)
            entries = []
            for cfg in configs(G, T, D):
                us = time_config(torch, binding, (q, k, v, out, lse), shape, D, bool(causal), cfg,
                                 args.repeats, stream)
                eo, el = check_rows(torch, out, lse, D, ref)
                entries.append((cfg, us, eo, el))
                print(f"D={D} causal={causal} large={large} {shape} cfg={cfg}: {us:9.2f} us "
                      f"{f / us / 1e6:7.1f} TFLOP/s  err O {eo:.2e} lse {el:.2e}", flush=True)
                if eo > 2e-2 or el > 2e-2:
                    print(f"parity FAILED for {cfg}", file=sys.stderr)
                    return 1
            results[(D, causal, large)] = entries
            best = min(entries, key=lambda e: e[1])
            rules.append((D, causal, large) + best[0])
        del q, k, v, out, lse
        torch.cuda.empty_cache()

    write_table(out_dir / "tile_table.inc", rules)
    write_report(out_dir / "tile_sweep_attn_fwd_bf16.md", results, rules, props, cus,
                 args.repeats)
    print(f"wrote {out_dir}/tile_table.inc and {out_dir}/tile_sweep_attn_fwd_bf16.md")
    return 0


TABLE_HEAD = """\
// Tile configurations of the bf16 forward, one rule per (head size, causal,
// problem size).  Written by attention_flashattention_fwd_amd/autotune.py from
// its sweep on MI355X (every configuration timed on each benchmark shape; the
// fastest kept); the sweep's timings are in profiles/tile_sweep_attn_fwd_bf16.md.
// Regenerate with `python -m attention_flashattention_fwd_amd.autotune`.
//
// large: query rows per compute unit (B * Hq * Tq / CUs) of at least
// kLargeRowsPerCu.  Fields: D, causal, large, heads_per_workgroup (the most
// the GQA group allows, up to this), query_rows_per_wave, workgroups_per_cu,
// persistent.
constexpr TileRule kTileTable[] = {
"""


def write_table(path: Path, rules) -> None:
    order = sorted(rules, key=lambda r: (-r[0], -r[1], -r[2]))
    body = "".join("    {" + ", ".join(str(int(x)) for x in r) + "},\n" for r in order)
    path.write_text(TABLE_HEAD + body + "};\n")


def parse_table(text: str):
    """The rules of a tile_table.inc, as tuples of ints."""
    return sorted(tuple(int(x) for x in m.group(1).split(","))
                  for m in re.finditer(r"^\s*\{([\d, ]+)\},\s*$", text, re.M))


def write_report(path: Path, results, rules, props, cus, repeats) -> None:
    lines = [
        "# Tile-configuration sweep of the bf16 attention forward (MI355X, gfx950)",
        "",
        f"Device: {props.name}, {cus} compute units.  Each configuration: 0.15 s of warm-up "
        f"launches, then the median of {repeats} batches of back-to-back launches timed with "
        "HIP events on the launch stream; every timed output checked against the fp64 oracle "
        "on 48 sampled rows (max-abs error of O and lse, bar 2e-2).  Inputs N(0,1) bf16 drawn "
        "on the GPU.  Configuration = (heads_per_workgroup, query_rows_per_wave, "
        "workgroups_per_cu, persistent).",
        "",
        "Command (from the repository root): `python -m attention_flashattention_fwd_amd.autotune`",
        "",
    ]
    for (D, causal, large), entries in sorted(results.items(), key=lambda kv: (-kv[0][0],
                                                                               -kv[0][1],
                                                                               -kv[0][2])):
        B, Hq, Hkv, T = SHAPES[(D, large)]
        f = flops(B, Hq, T, D, causal)
        best = min(entries, key=lambda e: e[1])
        lines += [f"## D={D}, causal={causal}, {'large' if large else 'small'}: B={B} Hq={Hq} "
                  f"Hkv={Hkv} T={T}", "",
                  "| configuration | us per launch | TFLOP/s | % of peak | max err O | max err lse |",
                  "|---|---|---|---|---|---|"]
        for cfg, us, eo, el in sorted(entries, key=lambda e: e[1]):
            mark = " **winner**" if cfg == best[0] else ""
            tf = f / us / 1e6
            lines.append(f"| {cfg}{mark} | {us:.2f} | {tf:.1f} | {100 * tf / PEAK_BF16_TFLOPS:.2f} "
                         f"| {eo:.2e} | {el:.2e} |")
        lines.append("")
    lines += ["## Rules written to csrc/tile_table.inc", "",
              "machine-readable (D, causal, large, heads_per_workgroup, query_rows_per_wave, "
              "workgroups_per_cu, persistent):", ""]
    lines += ["    rule: " + ", ".join(str(int(x)) for x in r)
              for r in sorted(rules, key=lambda r: (-r[0], -r[1], -r[2]))]
    path.write_text("\n".join(lines) + "\n")


if __name__ == "__main__":
    sys.exit(main())
